// Decode rows (one query token per sequence): split-K paged attention plus a
// log-sum-exp merge of the splits.
//
// What is computed is the exact softmax attention of "Under the Hood: Flash
// Attention" (Text Generation Inference page): a running max m, a running sum
// l of exponentials and an output accumulator rescaled by exp(m_old - m_new)
// whenever the max grows, finished by O / l.  The same rescale identity
// merges partial (O, m, l) triples computed over disjoint key ranges, which is
// what the merge kernel does across splits.  Keys and values are reached
// through the sequence's block table ("Under the Hood: PagedAttention").
//
// Work decomposition (gfx950, 64-lane waves):
//   grid  = (split, kv head, sequence); block = 4 waves.
//   Every wave walks its own 64-token tiles of the split (tiles w, w+4, ...):
//     * the K tile is staged through LDS with coalesced 16-byte loads (16
//       lanes per 256-byte row) and read back one row per lane (XOR-swizzled
//       16-byte chunks, conflict-free), so lane t owns token t;
//     * QK: lane t forms the G dot products of its key with the G query heads
//       of the GQA group (packed bf16 dot2 with fp32 accumulation) -- all G
//       heads share the one K read, and no cross-lane reduction is needed;
//     * softmax: per head, a wave max (shuffles), exp2, per-lane partial sums;
//       probabilities go to LDS;
//     * PV: lane d owns two output dims of all G heads; each V row is one
//       coalesced 256-byte load (4 bytes per lane), weights are LDS broadcasts.
//   The 4 waves' (O, m, l) are combined through LDS; a sequence with one split
//   writes bf16 output directly, otherwise fp32 partials go to the workspace.
#include "common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kTile = 64;     // tokens per wave iteration (one per lane in the QK step)
constexpr int kWaves = 4;     // waves per workgroup; each walks its own tiles of the split
constexpr int kVPL = 4;       // V elements per lane per load (8-byte loads)

// 16-byte / 8-byte vector types for the V loads.
template <int N> struct VecOf;
template <> struct VecOf<8> { typedef uint4 T; };
template <> struct VecOf<4> { typedef uint2 T; };

__device__ __forceinline__ void unpack(const uint4& v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}
__device__ __forceinline__ void unpack(const uint2& v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
}

template <int D, int G, int BS>
__global__ __launch_bounds__(kWaves * kWave) void decode_split_kernel(AttnParams p) {
  constexpr int CH = D / 8;              // 16-byte chunks per K row
  constexpr int VPL = kVPL;
  constexpr int LPR = D / VPL;           // lanes per V row
  constexpr int TPI = kWave / LPR;       // V rows per wave-wide load
  constexpr int NV = kTile / TPI;        // V loads per lane per tile
  constexpr int NBT = kTile / BS;        // blocks spanned by one tile
  typedef typename VecOf<VPL>::T VT;
  static_assert(BS % TPI == 0 && kTile % BS == 0, "rows of one V load must share a block");

  constexpr int GP = G < 4 ? 4 : G;      // heads padded to a float4
  __shared__ float4 ptile[kWaves][kTile][GP / 4];   // softmax weights of the current tile
  __shared__ float sm_o[kWaves][G][D];
  __shared__ float sm_ml[kWaves][G][2];

  const int split = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int row0 = p.qsl[s];
  if (p.qsl[s + 1] - row0 != 1) return;          // not a decode row
  if (row0 < 0 || row0 >= p.num_q_tokens) return;
  // lengths beyond what the table row can map are clamped (caller error)
  const int L = min(p.seq_lens[s], p.max_blocks * BS);
  const int t_begin = split * p.split_tokens;
  if (t_begin >= L) return;                      // split past the end of the sequence
  const int t_end = min(t_begin + p.split_tokens, L);
  const int nsplit = (L + p.split_tokens - 1) / p.split_tokens;

  const int lane = threadIdx.x & (kWave - 1);
  const int w = uniform(threadIdx.x / kWave);
  const int Hq = p.Hkv * G;
  const int* bt_row = p.block_tables + (size_t)s * p.max_blocks;
  const size_t row_stride = (size_t)p.Hkv * D;   // elements per pool slot
  const uint16_t* kbase = p.k_cache + (size_t)h * D;
  const uint16_t* vbase = p.v_cache + (size_t)h * D;
  const uint4* qv = reinterpret_cast<const uint4*>(p.q + ((size_t)row0 * Hq + (size_t)h * G) * D);
  const float c = p.scale_log2;
  const int vt = lane / LPR;                     // V token group of this lane
  const int vd = (lane % LPR) * VPL;             // first V dim of this lane
  const int nblocks = (unsigned)p.num_blocks > 0x7fffffffu ? 0x7fffffff : (int)p.num_blocks;

  float m_run[G], l_part[G], o[G][VPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY; l_part[g] = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) o[g][j] = 0.f;
  }

  const size_t blk_bytes = (size_t)BS * row_stride * 2;
  const uint32_t row_bytes = (uint32_t)(row_stride * 2);
  const int ntiles = (t_end - t_begin + kTile - 1) / kTile;     // tiles of the split
  for (int tile = w; tile < ntiles; tile += kWaves) {
    const int ts = t_begin + tile * kTile;
    const int nvalid = min(kTile, t_end - ts);

    // Block-table entries of the tile (wave-uniform scalar loads).  Entries past the end,
    // or outside the pool, become block 0: a safe address whose rows the masks ignore.
    int bts[NBT];
#pragma unroll
    for (int j = 0; j < NBT; ++j) {
      const int b = (j * BS < nvalid) ? bt_row[uniform((ts + j * BS) / BS)] : 0;
      bts[j] = (unsigned)b < (unsigned)nblocks ? b : 0;
    }

    // ---- issue all loads of the tile: K (lane = token, whole row), V (lane = VPL dims) ----
    uint4 kreg[CH];
    {
      int blk = bts[0];
#pragma unroll
      for (int j = 1; j < NBT; ++j) if (lane / BS == j) blk = bts[j];
      const uint4* src = reinterpret_cast<const uint4*>(
          reinterpret_cast<const char*>(kbase) + (size_t)blk * blk_bytes + (uint32_t)(lane % BS) * row_bytes);
#pragma unroll
      for (int cc = 0; cc < CH; ++cc) kreg[cc] = src[cc];
    }
    VT vreg[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const char* base = reinterpret_cast<const char*>(vbase) + (size_t)bts[(TPI * i) / BS] * blk_bytes;
      const uint32_t off = (uint32_t)((TPI * i) % BS + vt) * row_bytes + (uint32_t)vd * 2;
      vreg[i] = *reinterpret_cast<const VT*>(base + off);
    }

    // ---- QK: lane owns token ts + lane; q sits in scalar registers ----
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
    // q is re-read from the scalar cache every tile: an opaque zero offset stops the
    // compiler from hoisting G*D/2 values out of the loop into vector registers.
    int zero;
    asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
    // constant address space: uniform loads from it are always scalar (s_load)
    typedef const __attribute__((address_space(4))) uint32_t cu32;
    cu32* qt = (cu32*)(qv + zero);
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      const uint4 kk = kreg[cc];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        cu32* qq = qt + 4 * (g * CH + cc);
        float a = acc[g];
        a = dot2_bf16(qq[0], kk.x, a);
        a = dot2_bf16(qq[1], kk.y, a);
        a = dot2_bf16(qq[2], kk.z, a);
        a = dot2_bf16(qq[3], kk.w, a);
        acc[g] = a;
      }
    }

    // ---- online softmax (exp2 domain) ----
    const bool valid = lane < nvalid;
    float alpha[G];
    float pe[GP];
#pragma unroll
    for (int g = G; g < GP; ++g) pe[g] = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sc = valid ? acc[g] * c : -INFINITY;
      const float mn = fmaxf(m_run[g], wave_max(sc));   // finite: lane 0 is always valid
      alpha[g] = exp2f(m_run[g] - mn);                  // 0 on the first tile
      pe[g] = valid ? exp2f(sc - mn) : 0.f;
      l_part[g] = l_part[g] * alpha[g] + pe[g];
      m_run[g] = mn;
    }
#pragma unroll
    for (int g4 = 0; g4 < GP / 4; ++g4)
      ptile[w][lane][g4] = make_float4(pe[4 * g4], pe[4 * g4 + 1], pe[4 * g4 + 2], pe[4 * g4 + 3]);
    wave_lds_sync();

    // ---- PV: lane owns VPL dims of every TPI-th token ----
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < VPL; ++j) o[g][j] *= alpha[g];
    const int vlim = nvalid - vt;                       // token slot i is valid iff TPI*i < vlim
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      // keep the weight reads next to their use (hoisting all of them costs registers)
      if (i % 4 == 0) __builtin_amdgcn_sched_barrier(0);
      const int r = TPI * i + vt;
      float vf[VPL];
      unpack(vreg[i], vf);
      if (TPI * i < vlim) {} else {                     // rows past the end may hold NaN; weight is 0
#pragma unroll
        for (int j = 0; j < VPL; ++j) vf[j] = 0.f;
      }
      float pw[GP];
#pragma unroll
      for (int g4 = 0; g4 < GP / 4; ++g4) {
        const float4 t4 = ptile[w][r][g4];
        pw[4 * g4] = t4.x; pw[4 * g4 + 1] = t4.y; pw[4 * g4 + 2] = t4.z; pw[4 * g4 + 3] = t4.w;
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < VPL; ++j) o[g][j] = fmaf(pw[g], vf[j], o[g][j]);
    }
    wave_lds_sync();
  }

  // ---- combine: token groups inside the wave, then the waves ----
  float l_tot[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l_tot[g] = wave_sum(l_part[g]);
#pragma unroll
    for (int msk = LPR; msk < kWave; msk *= 2)
#pragma unroll
      for (int j = 0; j < VPL; ++j) o[g][j] += __shfl_xor(o[g][j], msk, kWave);
  }
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < VPL; ++j) sm_o[w][g][vd + j] = o[g][j];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) { sm_ml[w][g][0] = m_run[g]; sm_ml[w][g][1] = l_tot[g]; }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int g = e / D, d = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm_ml[ww][g][0]);
    float O = 0.f, Ls = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = exp2f(sm_ml[ww][g][0] - M);   // 0 for a wave without tokens
      Ls = fmaf(f, sm_ml[ww][g][1], Ls);
      O = fmaf(f, sm_o[ww][g][d], O);
    }
    const int qh = h * G + g;
    if (nsplit == 1) {
      p.out[((size_t)row0 * Hq + qh) * D + d] = f32_to_bf16_rne(O / Ls);
    } else {
      const size_t idx = ((size_t)s * Hq + qh) * p.max_splits + split;
      p.ws_o[idx * D + d] = O;
      if (d == 0) { p.ws_m[idx] = M; p.ws_l[idx] = Ls; }
    }
  }
}

// Log-sum-exp merge of the splits of one (decode sequence, query head):
// out = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j with M = max_j m_j.
template <int D>
__global__ __launch_bounds__(D) void merge_kernel(AttnParams p) {
  const int s = blockIdx.x, qh = blockIdx.y, d = threadIdx.x;
  const int row0 = p.qsl[s];
  if (p.qsl[s + 1] - row0 != 1) return;
  if (row0 < 0 || row0 >= p.num_q_tokens) return;
  const int L = min(p.seq_lens[s], p.max_blocks * p.bs);
  const int nsplit = (L + p.split_tokens - 1) / p.split_tokens;
  if (nsplit <= 1) return;                       // written directly by the split kernel
  const size_t base = ((size_t)s * p.Hq + qh) * p.max_splits;
  float M = -INFINITY;
  for (int j = 0; j < nsplit; ++j) M = fmaxf(M, p.ws_m[base + j]);
  float O = 0.f, Ls = 0.f;
  for (int j = 0; j < nsplit; ++j) {
    const float f = exp2f(p.ws_m[base + j] - M);
    Ls = fmaf(f, p.ws_l[base + j], Ls);
    O = fmaf(f, p.ws_o[(base + j) * D + d], O);
  }
  p.out[((size_t)row0 * p.Hq + qh) * D + d] = f32_to_bf16_rne(O / Ls);
}

template <int D, int G, int BS>
hipError_t launch_decode_t(const AttnParams& p, hipStream_t stream) {
  dim3 grid(p.max_splits, p.Hkv, p.num_seqs);
  hipLaunchKernelGGL((decode_split_kernel<D, G, BS>), grid, dim3(kWaves * kWave), 0, stream, p);
  return hipGetLastError();
}

template <int D, int G>
hipError_t dispatch_bs(const AttnParams& p, hipStream_t stream) {
  switch (p.bs) {
    case 8: return launch_decode_t<D, G, 8>(p, stream);
    case 16: return launch_decode_t<D, G, 16>(p, stream);
    case 32: return launch_decode_t<D, G, 32>(p, stream);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t dispatch_g(const AttnParams& p, hipStream_t stream) {
  switch (p.Hq / p.Hkv) {
    case 1: return dispatch_bs<D, 1>(p, stream);
    case 2: return dispatch_bs<D, 2>(p, stream);
    case 4: return dispatch_bs<D, 4>(p, stream);
    case 8: return dispatch_bs<D, 8>(p, stream);
    case 16: return dispatch_bs<D, 16>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_supported(int D, int G, int bs) {
  return (D == 64 || D == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16) &&
         (bs == 8 || bs == 16 || bs == 32);
}

hipError_t launch_decode(const AttnParams& p, hipStream_t stream) {
  if (p.D == 128) return dispatch_g<128>(p, stream);
  if (p.D == 64) return dispatch_g<64>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const AttnParams& p, hipStream_t stream) {
  dim3 grid(p.num_seqs, p.Hq);
  if (p.D == 128) hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(128), 0, stream, p);
  else if (p.D == 64) hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(64), 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
