// Chunked-prefill rows (q_s > 1): causal attention of a chunk of new tokens
// over the sequence's cached prefix and over the chunk itself, on the bf16
// matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// The computation is the tiled exact attention of "Under the Hood: Flash
// Attention" (Text Generation Inference page) -- scores of a query tile
// against one K tile at a time, running row max and row sum, output rescaled
// when the max grows -- applied to rows that continue an existing prefix
// ("Advanced Pattern: Chunked Prefill"): row j of a chunk of q_s tokens in a
// sequence of L tokens sits at position L - q_s + j and sees keys 0..that
// position, gathered through the block table ("Under the Hood: PagedAttention").
//
// Layout choices for gfx950:
//   * A workgroup (4 waves) owns 128 (query row, query head) pairs of one KV
//     head: the G heads of a GQA group are packed into the M dimension, so
//     each K/V tile is loaded once for all of them.  Wave w owns 32 pairs.
//   * Scores are computed transposed, S^T = K Q^T (keys x pairs): A = K rows
//     (16-byte chunks from LDS), B = Q rows (registers, loaded once).  In the
//     32x32 accumulator each lane then holds one pair's column, so the row
//     max / row sum need a single cross-lane exchange (lane ^ 32).
//   * The output is computed transposed too, O^T = V^T P^T: the B operand P^T
//     is exactly the score accumulator converted to bf16 in place (no LDS
//     round trip); the A operand V^T is read from an LDS copy of the V tile
//     that is stored transposed ([dim][key], rows padded to 68 keys).
//   * K/V tiles are 64 keys, gathered from the paged pool block by block.
//   * Keys past the sequence end are zero-filled in LDS (V especially: a
//     masked weight of 0 times a NaN in an unused slot would poison the sum).
//   * Software pipeline: the next K/V tile is loaded into registers while the
//     current one is multiplied out of LDS.
//   * A one-block planner kernel lists the (sequence, row tile) items of the
//     prefill sequences in the workspace (later row tiles first: they see the
//     most keys), so no workgroup is launched for decode rows; workgroup ids
//     are remapped so that consecutive items of one (sequence, KV head) run on
//     the same XCD and share its L2.
#include "common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kWavesP = 4;
constexpr int kPairsPerWave = 32;
constexpr int kPairsPerBlock = kWavesP * kPairsPerWave;   // 128
static_assert(kPairsPerBlock == kPrefillPairs, "planner and kernel agree on the row tile");
constexpr int kKT = 64;                                    // keys per tile
constexpr int kVTRow = kKT + 4;                            // padded row of the transposed V tile

// Lists the prefill work items (sequence, row tile) of one call: a sequence
// with q_s > 1 rows has ceil(q_s / rows_per_tile) row tiles, emitted last tile
// first.  One block; sequences are scanned in chunks of the block size.
constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(const int32_t* __restrict__ qsl, int num_seqs,
                                                                    int rows_per_tile, int2* __restrict__ items,
                                                                    int* __restrict__ count, int capacity) {
  __shared__ int wave_tot[kPlanThreads / kWave];
  __shared__ int base_sh;
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  if (t == 0) base_sh = 0;
  __syncthreads();
  for (int s0 = 0; s0 < num_seqs; s0 += kPlanThreads) {
    const int s = s0 + t;
    int nt = 0;
    if (s < num_seqs) {
      const int q = qsl[s + 1] - qsl[s];
      if (q > 1) nt = (q + rows_per_tile - 1) / rows_per_tile;
    }
    // inclusive scan inside the wave, then across waves
    int incl = nt;
#pragma unroll
    for (int d = 1; d < kWave; d *= 2) {
      const int y = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += y;
    }
    if (lane == kWave - 1) wave_tot[w] = incl;
    __syncthreads();
    int before = base_sh;
    for (int i = 0; i < w; ++i) before += wave_tot[i];
    const int off = before + incl - nt;
    for (int k = 0; k < nt; ++k)
      if (off + k < capacity) items[off + k] = make_int2(s, nt - 1 - k);
    __syncthreads();
    if (t == kPlanThreads - 1) base_sh = off + nt;
    __syncthreads();
  }
  if (t == 0) *count = min(base_sh, capacity);
}

// Workgroup ids are handed to the 8 XCDs round-robin (id % 8).  This maps them
// to logical ids so that XCD x runs the contiguous logical range
// [x * n / 8, (x + 1) * n / 8); n is a multiple of 8.
__device__ __forceinline__ int xcd_logical_id(int id, int n) {
  constexpr int kXcd = 8;
  return (id % kXcd) * (n / kXcd) + id / kXcd;
}

template <int D, int G>
__global__ __launch_bounds__(256, 2) void prefill_kernel(AttnParams p) {
  constexpr int CH = D / 8;          // 16-byte chunks per K/V row
  constexpr int KS = D / 16;         // k-steps of the QK product
  constexpr int DT = D / 32;         // 32-wide dim tiles of the output
  constexpr int ROWS = kPairsPerBlock / G;   // query rows per workgroup

  __shared__ uint4 ks_tile[kKT][CH];                    // K tile, row-major, chunk-swizzled
  __shared__ __attribute__((aligned(16))) uint32_t vt_tile[D][kVTRow / 2];   // V^T tile, bf16 pairs along keys

  // logical id -> (KV head, work item); items past the planner's count do nothing
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int h = lid / p.plan_stride, item = lid % p.plan_stride;
  if (h >= p.Hkv || item >= *p.plan_count || item >= p.plan_capacity) return;
  const int2 it = p.plan_items[item];
  const int s = it.x, mt = it.y;
  const int row0 = p.qsl[s];
  const int qn = p.qsl[s + 1] - row0;
  if (qn <= 1) return;                           // decode rows are handled elsewhere
  const int j0 = mt * ROWS;
  if (j0 >= qn) return;
  if (row0 < 0 || row0 + qn > p.num_q_tokens) return;
  const int L = min(p.seq_lens[s], p.max_blocks * p.bs);   // clamp a length the table cannot map
  const int prior = L - qn;
  const int j1 = min(j0 + ROWS, qn);
  const int key_end = prior + j1;                // keys [0, key_end) are needed by this block

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = uniform(tid / kWave);
  const int Hq = p.Hkv * G;
  const int* bt_row = p.block_tables + (size_t)s * p.max_blocks;
  const size_t row_stride = (size_t)p.Hkv * D;
  const uint16_t* kbase = p.k_cache + (size_t)h * D;
  const uint16_t* vbase = p.v_cache + (size_t)h * D;
  const int BS = p.bs;

  // ---- this lane's pair (B-operand column / accumulator column) ----
  const int n = lane & 31;                       // column inside the wave's 32 pairs
  const int kg = lane >> 5;                      // k-group: which 8 of each 16-wide k step
  const int pair = w * kPairsPerWave + n;        // 0..127
  const int jrow = j0 + pair / G;
  const int gq = pair % G;
  const bool pair_valid = jrow < j1;
  // last key this pair may attend (inclusive); invalid pairs see only key 0
  const int lim = pair_valid ? prior + jrow : 0;
  // wave-level bounds of the causal limits (uniform)
  const int wj_lo = j0 + (w * kPairsPerWave) / G;
  const int wave_lim_min = prior + min(wj_lo, j1 - 1);
  const int wave_lim_max = prior + min(j0 + (w * kPairsPerWave + kPairsPerWave - 1) / G, j1 - 1);
  const bool wave_active = wj_lo < j1;

  // ---- Q as the B operand: 8 consecutive dims per k step ----
  bf16x8 qreg[KS];
  {
    const uint16_t* qp = p.q + ((size_t)(row0 + (pair_valid ? jrow : j0)) * Hq + (size_t)h * G + gq) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (pair_valid) v = *reinterpret_cast<const uint4*>(qp + ks * 16 + kg * 8);
      qreg[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  floatx16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  float m_run = -INFINITY, l_part = 0.f;
  const float c = p.scale_log2;

  auto tile_compute = [&](int kb) {
    if (!wave_active || kb > wave_lim_max) return;     // nothing unmasked for this wave

    // ---- S^T = K Q^T for the two 32-key halves of the tile ----
    floatx16 sacc[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[hf][i] = 0.f;
      const int r = hf * 32 + n;                     // key row this lane feeds as A
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int cc = ks * 2 + kg;
        const uint4 kv = ks_tile[r][cc ^ (r % CH)];
        sacc[hf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv), qreg[ks],
                                                           sacc[hf], 0, 0, 0);
      }
    }

    // ---- mask, online softmax (exp2 domain) ----
    const bool need_mask = kb + kKT - 1 > wave_lim_min;
    float tmax = -INFINITY;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = sacc[hf][i] * c;
        if (need_mask) {
          const int key = kb + hf * 32 + 8 * (i / 4) + 4 * kg + (i % 4);
          if (key > lim) v = -INFINITY;
        }
        sacc[hf][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float mn = fmaxf(m_run, tmax);        // finite: key 0 of the first tile is visible to all
    const float alpha = fast_exp2(m_run - mn);
    m_run = mn;
    float psum = 0.f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(sacc[hf][i] - mn);   // 2^-inf = 0 for masked keys
        sacc[hf][i] = e;
        psum += e;
      }
    l_part = l_part * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;

    // ---- O^T += V^T P^T over four 16-key steps ----
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int hf = kk >> 1, part = kk & 1;
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[i] = (__bf16)sacc[hf][part * 8 + i];
      const int key_lo = kk * 16 + 4 * kg;            // keys key_lo..+3 and key_lo+8..+11
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = dt * 32 + n;
        const uint2 lo = *reinterpret_cast<const uint2*>(&vt_tile[d][key_lo / 2]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&vt_tile[d][(key_lo + 8) / 2]);
        const uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb, oacc[dt],
                                                           0, 0, 0);
      }
    }
    };

  // ---- tile staging: global -> registers (prefetch) -> LDS ----
  constexpr int NK = kKT * CH / 256;             // K chunks per thread
  constexpr int NV = (kKT / 2) * CH / 256;       // V (key pair, chunk) items per thread
  uint4 kpre[NK], vpa[NV], vpb[NV];
  auto load_tile = [&](int kb) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int e = tid + 256 * i, r = e / CH, cc = e % CH, tok = kb + r;
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (tok < key_end) {
        const int blk = bt_row[tok / BS];
        if ((unsigned)blk < (unsigned)p.num_blocks)
          val = *reinterpret_cast<const uint4*>(kbase + ((size_t)blk * BS + tok % BS) * row_stride + cc * 8);
      }
      kpre[i] = val;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = tid + 256 * i, r2 = e / CH, cc = e % CH;
      const int t0 = kb + 2 * r2, t1 = t0 + 1;
      uint4 a = make_uint4(0u, 0u, 0u, 0u), b = make_uint4(0u, 0u, 0u, 0u);
      if (t0 < key_end) {
        const int blk = bt_row[t0 / BS];
        if ((unsigned)blk < (unsigned)p.num_blocks)
          a = *reinterpret_cast<const uint4*>(vbase + ((size_t)blk * BS + t0 % BS) * row_stride + cc * 8);
      }
      if (t1 < key_end) {
        const int blk = bt_row[t1 / BS];
        if ((unsigned)blk < (unsigned)p.num_blocks)
          b = *reinterpret_cast<const uint4*>(vbase + ((size_t)blk * BS + t1 % BS) * row_stride + cc * 8);
      }
      vpa[i] = a;
      vpb[i] = b;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int e = tid + 256 * i, r = e / CH, cc = e % CH;
      ks_tile[r][cc ^ (r % CH)] = kpre[i];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = tid + 256 * i, r2 = e / CH, cc = e % CH;
      const uint32_t aw[4] = {vpa[i].x, vpa[i].y, vpa[i].z, vpa[i].w};
      const uint32_t bw[4] = {vpb[i].x, vpb[i].y, vpb[i].z, vpb[i].w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int d = cc * 8 + 2 * x;
        vt_tile[d][r2] = (aw[x] & 0xffffu) | (bw[x] << 16);
        vt_tile[d + 1][r2] = (aw[x] >> 16) | (bw[x] & 0xffff0000u);
      }
    }
  };

  load_tile(0);
  store_tile();
  __syncthreads();
  for (int kb = 0; kb < key_end; kb += kKT) {
    const bool has_next = kb + kKT < key_end;
    if (has_next) load_tile(kb + kKT);           // in flight while this tile is multiplied
    tile_compute(kb);
    __syncthreads();                             // every wave is done with this tile
    if (has_next) {
      store_tile();
      __syncthreads();
    }
  }
  // ---- finish: O / l, bf16 out ----
  if (!pair_valid) return;
  const float l_tot = l_part + __shfl_xor(l_part, 32, kWave);
  const float inv = 1.f / l_tot;
  uint16_t* op = p.out + ((size_t)(row0 + jrow) * Hq + (size_t)h * G + gq) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = dt * 32 + 8 * q4 + 4 * kg;
      const uint32_t w0 = (uint32_t)f32_to_bf16_rne(oacc[dt][q4 * 4 + 0] * inv) |
                          ((uint32_t)f32_to_bf16_rne(oacc[dt][q4 * 4 + 1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16_rne(oacc[dt][q4 * 4 + 2] * inv) |
                          ((uint32_t)f32_to_bf16_rne(oacc[dt][q4 * 4 + 3] * inv) << 16);
      *reinterpret_cast<uint2*>(op + d) = make_uint2(w0, w1);
    }
}

template <int D>
hipError_t dispatch_g(const AttnParams& p, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  const int rows = kPairsPerBlock / G;
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p.qsl, p.num_seqs, rows,
                     p.plan_items, p.plan_count, p.plan_capacity);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one workgroup per (KV head, possible item); rounded up to the 8 XCDs
  const int64_t n = ((int64_t)p.Hkv * p.plan_stride + 7) / 8 * 8;
  dim3 grid((unsigned)n);
  switch (G) {
    case 1: hipLaunchKernelGGL((prefill_kernel<D, 1>), grid, dim3(256), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<D, 2>), grid, dim3(256), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<D, 4>), grid, dim3(256), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<D, 8>), grid, dim3(256), 0, stream, p); break;
    case 16: hipLaunchKernelGGL((prefill_kernel<D, 16>), grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool prefill_supported(int D, int G, int bs) {
  return (D == 64 || D == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16) && bs > 0;
}

hipError_t launch_prefill(const AttnParams& p, hipStream_t stream) {
  if (p.max_query_len <= 1) return hipSuccess;
  if (p.D == 128) return dispatch_g<128>(p, stream);
  if (p.D == 64) return dispatch_g<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
