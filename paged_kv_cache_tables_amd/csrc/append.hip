// kv_append: scatter new K/V rows into their pool slots (bit copy).
//
// "Under the Hood: PagedAttention" (Text Generation Inference page): a new
// token's K/V pair is appended at its sequence's next position, inside the
// physical block the sequence's block table maps that position to.  With the
// pool laid out [num_blocks, block_size, kv_heads, head_dim], the flat row of
// slot s is simply s, so the append is a row scatter: every 16-byte chunk of
// new row i goes to chunk c of pool row slot_mapping[i].
#include "common.h"
#include "kernels.h"

namespace pkv {

// One thread per 16-byte chunk of K or V; consecutive threads cover
// consecutive chunks of one row, so loads and stores are fully coalesced.
__global__ __launch_bounds__(256) void append_kernel(const uint4* __restrict__ k_new,
                                                     const uint4* __restrict__ v_new,
                                                     const int64_t* __restrict__ slots,
                                                     int64_t num_tokens, uint4* __restrict__ k_cache,
                                                     uint4* __restrict__ v_cache, int64_t num_slots,
                                                     int row_chunks) {
  const int64_t per_token = 2 * (int64_t)row_chunks;
  const int64_t total = num_tokens * per_token;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = idx / per_token;
    const int rem = (int)(idx - i * per_token);
    const int which = rem >= row_chunks;          // 0 = K, 1 = V
    const int c = rem - which * row_chunks;
    const int64_t slot = slots[i];
    if (slot < 0 || slot >= num_slots) continue;  // padding row, or outside the pool
    const uint4* src = which ? v_new : k_new;
    uint4* dst = which ? v_cache : k_cache;
    dst[slot * row_chunks + c] = src[i * row_chunks + c];
  }
}

hipError_t launch_append(const void* k_new, const void* v_new, const int64_t* slots, int64_t num_tokens,
                         void* k_cache, void* v_cache, int64_t num_slots, int row_chunks,
                         hipStream_t stream) {
  const int64_t total = num_tokens * 2 * (int64_t)row_chunks;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;  // grid-stride loop covers the rest
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     (const uint4*)k_new, (const uint4*)v_new, slots, num_tokens, (uint4*)k_cache,
                     (uint4*)v_cache, num_slots, row_chunks);
  return hipGetLastError();
}

// ---- whole-block copies (copy-on-write of a shared block) ----
// Workgroup i copies pair i's block in K and in V, 16 bytes per thread and step.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                                                          const int32_t* __restrict__ src,
                                                          const int32_t* __restrict__ dst, int64_t num_blocks,
                                                          int64_t chunks16) {
  const int32_t s = src[blockIdx.x], d = dst[blockIdx.x];
  if (s == d || s < 0 || d < 0 || s >= num_blocks || d >= num_blocks) return;
  const uint4* ks = k_cache + (int64_t)s * chunks16;
  const uint4* vs = v_cache + (int64_t)s * chunks16;
  uint4* kd = k_cache + (int64_t)d * chunks16;
  uint4* vd = v_cache + (int64_t)d * chunks16;
  for (int64_t c = threadIdx.x; c < chunks16; c += blockDim.x) {
    kd[c] = ks[c];
    vd[c] = vs[c];
  }
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst, int n_pairs,
                              int64_t num_blocks, int64_t chunks16, hipStream_t stream) {
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)n_pairs), dim3(256), 0, stream, (uint4*)k_cache,
                     (uint4*)v_cache, src, dst, num_blocks, chunks16);
  return hipGetLastError();
}

// ---- E4M3 pools ----
//
// An 8-bit cache stores, for each value x of a new row, the E4M3 code nearest to
// y = x / scale ("How to Speed Up LLM Inference", "Quantization: move fewer bytes":
// values in few bits with a shared scale factor; "The KV cache ...": an FP8 cache halves
// the bytes per token).  y is the correctly rounded float32 quotient; the code is the
// nearest E4M3 value (4 exponent bits, bias 7, 3 mantissa bits, no infinities,
// S.1111.111 = NaN), ties to the even code; |y| >= 448 gives the largest finite code.

// Nearest E4M3 code of a float32 value (sign copied; NaN input saturates like a large value).
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t code;
  if (!(a < 448.f)) {
    code = 0x7Eu;                                        // 448
  } else if (a < 0x1p-6f) {
    // zero and subnormals are the multiples of 2^-9 below 2^-6: a * 512 is exact, and
    // rounding it to the nearest integer (ties to even) gives the code (8 = 2^-6, the
    // smallest normal, whose code is 0x08)
    code = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    const uint32_t ua = __float_as_uint(a);
    const uint32_t e = (ua >> 23) - 127u + 7u;           // E4M3 exponent field, 1..15
    const uint32_t mant = ua & 0x7FFFFFu;
    uint32_t c = (e << 3) | (mant >> 20);                // truncated to 3 mantissa bits
    const uint32_t rem = mant & 0xFFFFFu;                // the 20 dropped bits
    if (rem > 0x80000u || (rem == 0x80000u && (c & 1u))) c += 1u;   // a carry moves to the next binade
    code = c;                                            // a < 448 keeps it <= 0x7E
  }
  return code | sign;
}

// One thread per 16 codes (16 bytes) of a K or V row: 32 bytes of bf16 in, 16 bytes out.
__global__ __launch_bounds__(256) void append_fp8_kernel(const uint4* __restrict__ k_new,
                                                         const uint4* __restrict__ v_new,
                                                         const int64_t* __restrict__ slots,
                                                         int64_t num_tokens, uint4* __restrict__ k_cache,
                                                         uint4* __restrict__ v_cache, int64_t num_slots,
                                                         int row_chunks16, float k_scale, float v_scale) {
  const int64_t per_token = 2 * (int64_t)row_chunks16;
  const int64_t total = num_tokens * per_token;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = idx / per_token;
    const int rem = (int)(idx - i * per_token);
    const int which = rem >= row_chunks16;               // 0 = K, 1 = V
    const int c = rem - which * row_chunks16;
    const int64_t slot = slots[i];
    if (slot < 0 || slot >= num_slots) continue;         // padding row, or outside the pool
    const uint4* src = (which ? v_new : k_new) + (i * row_chunks16 + c) * 2;
    const float scale = which ? v_scale : k_scale;
    const uint4 in[2] = {src[0], src[1]};
    uint32_t out[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint4 h = in[w / 2];
      const uint32_t lo = (w % 2) ? h.z : h.x, hi = (w % 2) ? h.w : h.y;   // 4 bf16 values
      uint32_t packed = 0;
      const uint32_t b[4] = {lo << 16, lo & 0xFFFF0000u, hi << 16, hi & 0xFFFF0000u};
#pragma unroll
      for (int j = 0; j < 4; ++j) packed |= f32_to_e4m3(__uint_as_float(b[j]) / scale) << (8 * j);
      out[w] = packed;
    }
    (which ? v_cache : k_cache)[slot * row_chunks16 + c] = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

hipError_t launch_append_fp8(const void* k_new, const void* v_new, const int64_t* slots, int64_t num_tokens,
                             void* k_cache, void* v_cache, int64_t num_slots, int row_chunks16,
                             float k_scale, float v_scale, hipStream_t stream) {
  const int64_t total = num_tokens * 2 * (int64_t)row_chunks16;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;  // grid-stride loop covers the rest
  hipLaunchKernelGGL(append_fp8_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     (const uint4*)k_new, (const uint4*)v_new, slots, num_tokens, (uint4*)k_cache,
                     (uint4*)v_cache, num_slots, row_chunks16, k_scale, v_scale);
  return hipGetLastError();
}

}  // namespace pkv
