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

constexpr int kTile = 64;     // tokens per wave iteration (one per lane)
constexpr int kWaves = 4;

template <int D, int G, int BS>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(AttnParams p) {
  constexpr int CH = D / 8;            // 16-byte chunks per K row
  constexpr int RPI = kWave / CH;      // K rows staged per wave-wide load
  constexpr int NSTAGE = kTile / RPI;  // loads per lane per tile
  constexpr int LPT = D / 2;           // lanes per V row (4 bytes each)
  constexpr int TPS = kWave / LPT;     // V rows per wave-wide load
  static_assert(BS % RPI == 0 && BS % TPS == 0, "rows of one load must share a block");

  __shared__ uint4 ktile[kWaves][kTile][CH];
  __shared__ float ptile[kWaves][kTile][G];

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

  float m_run[G], l_part[G], o0[G], o1[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { m_run[g] = -INFINITY; l_part[g] = 0.f; o0[g] = 0.f; o1[g] = 0.f; }

  for (int ts = t_begin + w * kTile; ts < t_end; ts += kWaves * kTile) {
    const int nvalid = min(kTile, t_end - ts);

    // ---- stage the K tile: row r, chunk cc -> LDS [r][cc ^ (r % CH)] ----
#pragma unroll
    for (int it = 0; it < NSTAGE; ++it) {
      const int r = it * RPI + lane / CH;
      const int cc = lane % CH;
      const int first = ts + it * RPI;           // wave-uniform
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (first < t_end) {
        const int blk = bt_row[uniform(first / BS)];
        const int tok = ts + r;
        if (tok < t_end && (unsigned)blk < (unsigned)p.num_blocks)
          val = *reinterpret_cast<const uint4*>(kbase + ((size_t)blk * BS + tok % BS) * row_stride + cc * 8);
      }
      ktile[w][r][cc ^ (r % CH)] = val;
    }
    wave_lds_sync();

    // ---- QK: lane owns token `lane` ----
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      const uint4 kk = ktile[w][lane][cc ^ (lane % CH)];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint4 qq = qv[g * CH + cc];
        float a = acc[g];
        a = dot2_bf16(qq.x, kk.x, a);
        a = dot2_bf16(qq.y, kk.y, a);
        a = dot2_bf16(qq.z, kk.z, a);
        a = dot2_bf16(qq.w, kk.w, a);
        acc[g] = a;
      }
    }

    // ---- online softmax (exp2 domain) ----
    const bool valid = lane < nvalid;
    float alpha[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sc = valid ? acc[g] * c : -INFINITY;
      const float mn = fmaxf(m_run[g], wave_max(sc));   // finite: lane 0 is always valid
      alpha[g] = exp2f(m_run[g] - mn);                  // 0 on the first tile
      const float pe = valid ? exp2f(sc - mn) : 0.f;
      l_part[g] = l_part[g] * alpha[g] + pe;
      m_run[g] = mn;
      ptile[w][lane][g] = pe;
    }
    wave_lds_sync();

    // ---- PV: lane owns dims 2*(lane % LPT) and +1 ----
#pragma unroll
    for (int g = 0; g < G; ++g) { o0[g] *= alpha[g]; o1[g] *= alpha[g]; }
    const int dpair = lane % LPT;
    for (int rr = 0; rr < nvalid; rr += TPS) {
      const int r = rr + lane / LPT;
      const int blk = bt_row[uniform((ts + rr) / BS)];
      float v0 = 0.f, v1 = 0.f;
      if (r < nvalid && (unsigned)blk < (unsigned)p.num_blocks) {
        const int tok = ts + r;
        const uint32_t vw = *reinterpret_cast<const uint32_t*>(
            vbase + ((size_t)blk * BS + tok % BS) * row_stride + 2 * dpair);
        v0 = bf16_lo(vw);
        v1 = bf16_hi(vw);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pw = ptile[w][r][g];
        o0[g] = fmaf(pw, v0, o0[g]);
        o1[g] = fmaf(pw, v1, o1[g]);
      }
    }
    wave_lds_sync();
  }

  // ---- combine the 4 waves ----
  float l_tot[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l_tot[g] = wave_sum(l_part[g]);
    if (TPS > 1) {  // lanes of different token groups hold partial sums of the same dims
      o0[g] += __shfl_xor(o0[g], LPT, kWave);
      o1[g] += __shfl_xor(o1[g], LPT, kWave);
    }
  }
  __syncthreads();                                   // every wave is done with its K tiles
  float* sm_o = reinterpret_cast<float*>(&ktile[0][0][0]);   // [kWaves][G][D]
  float* sm_ml = sm_o + kWaves * G * D;                       // [kWaves][G][2]
  if (lane < LPT) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sm_o[(w * G + g) * D + 2 * lane] = o0[g];
      sm_o[(w * G + g) * D + 2 * lane + 1] = o1[g];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sm_ml[(w * G + g) * 2] = m_run[g];
      sm_ml[(w * G + g) * 2 + 1] = l_tot[g];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int g = e / D, d = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm_ml[(ww * G + g) * 2]);
    float O = 0.f, Ls = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = exp2f(sm_ml[(ww * G + g) * 2] - M);   // 0 for a wave without tokens
      Ls = fmaf(f, sm_ml[(ww * G + g) * 2 + 1], Ls);
      O = fmaf(f, sm_o[(ww * G + g) * D + d], O);
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
