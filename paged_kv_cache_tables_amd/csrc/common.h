// Device-side helpers shared by the gfx950 kernels of the paged attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include <type_traits>

namespace pkv {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// Two fp32 values rounded to the nearest bf16 (ties to even) and packed, lo in the low
// half (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// fp32 value rounded to the nearest bf16 (ties to even), returned as fp32.
__device__ __forceinline__ float round_bf16(float f) { return (float)(__bf16)f; }

// Two packed bf16 products accumulated in fp32: a.lo*b.lo + a.hi*b.hi + c.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

// 16 E4M3 codes (bytes of v, first code in the low byte of v.x) widened to 16 bf16 values:
// codes 0..7 into lo, 8..15 into hi, in order.  The conversion is exact (every E4M3 value,
// subnormals included, is a bf16 value); NaN codes give NaN.  v_cvt_scalef32_pk_bf16_fp8
// converts the two codes of one 16-bit half of a dword, here with scale 1.
__device__ __forceinline__ void e4m3x16_to_bf16(uint4 v, uint4& lo, uint4& hi) {
#define PKV_CVT2(w, high) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((w), 1.0f, (high)))
  lo = make_uint4(PKV_CVT2(v.x, false), PKV_CVT2(v.x, true), PKV_CVT2(v.y, false), PKV_CVT2(v.y, true));
  hi = make_uint4(PKV_CVT2(v.z, false), PKV_CVT2(v.z, true), PKV_CVT2(v.w, false), PKV_CVT2(v.w, true));
#undef PKV_CVT2
}

// Read of an int that is not written during the kernel, at a wave-uniform index, through
// the scalar data cache (s_load_dword): its wait is on the scalar counter, so it never waits
// for the wave's vector loads in flight.  Reads only; nothing is written this way.
typedef const __attribute__((address_space(4))) int const_int_as4;
__device__ __forceinline__ int load_uniform_int(const int* base, int idx) {
  return ((const_int_as4*)base)[idx];
}

// 2^x with the hardware instruction (results below 2^-126 flush to zero, which for
// softmax weights relative to a maximum weight of 1 is far below fp32 resolution).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Compile-time integers and an unrolled loop over them (indices stay constants, so
// register arrays indexed by them stay in registers).
template <int V> using IntC = std::integral_constant<int, V>;
template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IntC<I>());
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

// 16-byte global load with the streaming (non-temporal) hint: for data read once,
// so it does not displace reusable lines from the caches.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void* ptr) {
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// XOR swizzle of the 16-byte chunks of a row-major LDS tile with CH chunks per row
// (CH = 8 or 16): chunk c of row r sits at c ^ chunk_swizzle<CH>(r).  The LDS serves
// 256 bytes (64 banks) at a time; the pattern keeps the prefill read shapes
// conflict-free: one chunk of 16 consecutive rows (MFMA A operands of K), and the
// transposing reads of V, where 32 lanes cover 4 aligned rows x 4 adjacent chunks.
// For 256-byte rows: 0 4 8 12 2 6 10 14 1 5 9 13 3 7 11 15 over 16 consecutive rows.
template <int CH>
__device__ __forceinline__ int chunk_swizzle(int r) {
  static_assert(CH == 8 || CH == 16, "rows of 128 or 256 bytes");
  if constexpr (CH == 16) return 4 * (r & 3) + 2 * ((r >> 2) & 1) + ((r >> 3) & 1);
  else return (2 * (r & 3) + ((r >> 2) & 1)) & 7;
}

// Wave-uniform copy of a value (lands in a scalar register).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Orders LDS writes and reads of different lanes of one wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Cross-lane reductions over a whole 64-lane wave built from DPP row operations
// (quad swaps, half-row and row mirrors inside each 16-lane row, then row
// broadcasts 15 and 31 towards lane 63), finished by one readlane: the result
// is wave-uniform.  No LDS traffic.
template <typename Op>
__device__ __forceinline__ float wave_reduce_dpp(float v, Op op) {
  auto dpp = [](float x, int ctrl_sel) -> float {
    int xi = __float_as_int(x);
    int r;
    switch (ctrl_sel) {
      case 0: r = __builtin_amdgcn_update_dpp(xi, xi, 0xB1, 0xF, 0xF, false); break;   // quad_perm [1,0,3,2]
      case 1: r = __builtin_amdgcn_update_dpp(xi, xi, 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
      case 2: r = __builtin_amdgcn_update_dpp(xi, xi, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
      case 3: r = __builtin_amdgcn_update_dpp(xi, xi, 0x140, 0xF, 0xF, false); break;  // row_mirror
      case 4: r = __builtin_amdgcn_update_dpp(xi, xi, 0x142, 0xA, 0xF, false); break;  // row_bcast:15 -> rows 1,3
      default: r = __builtin_amdgcn_update_dpp(xi, xi, 0x143, 0xC, 0xF, false); break; // row_bcast:31 -> rows 2,3
    }
    return __int_as_float(r);
  };
  v = op(v, dpp(v, 0));
  v = op(v, dpp(v, 1));
  v = op(v, dpp(v, 2));
  v = op(v, dpp(v, 3));   // every lane holds its row's result
  v = op(v, dpp(v, 4));   // lanes of rows 1 and 3 also cover rows 0 and 2
  v = op(v, dpp(v, 5));   // lane 63 covers the wave
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

struct MaxOp { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };

__device__ __forceinline__ float wave_max(float v) { return wave_reduce_dpp(v, MaxOp()); }

}  // namespace pkv
