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
//     each K/V tile is loaded once for all of them.  Wave w owns 32 pairs (one
//     32-column MFMA group), which keeps a wave within 256 registers: two
//     workgroups share a CU, and one wave's softmax overlaps another's MFMAs.
//   * Scores are computed transposed, S^T = K Q^T (keys x pairs): A = K rows
//     (16-byte chunks from LDS), B = Q rows (registers, loaded once).  In the
//     32x32 accumulator each lane holds one pair's column, so the row max and
//     row sum need one exchange between the two half-waves.
//   * The output is computed transposed too, O^T = V^T P^T: the B operand P^T
//     is the score accumulator converted to bf16 in place; the A operand V^T
//     is read from the row-major V tile with ds_read_b64_tr_b16.
//   * K and V tiles (64 keys) are row-major in LDS with a XOR swizzle of the
//     16-byte chunks (row r's chunk c sits at c ^ chunk_swizzle(r), which
//     keeps the K operand reads and the transposing V reads conflict-free).  They are
//     filled by global-to-LDS loads (global_load_lds_dwordx4: no registers,
//     no LDS write instructions), double buffered: tile t is multiplied while
//     tile t+1 is in flight, with one barrier per tile.  Block-table entries
//     are read a tile ahead of the loads that use them.
//   * Tile rows past the needed keys hold a copy of the last needed key (a
//     finite value with weight 0), never an unused pool slot: a weight of 0
//     times a NaN left in such a slot would poison the sum.
//   * The running max is raised lazily: the output and row sum are rescaled
//     only when some row's max grows by more than 2^8 (in the exp2 domain).
//     Until then weights are taken against the stale max and stay below 2^8,
//     so the result is the same softmax (the common factor cancels in O / l);
//     only rounding differs, and bf16 keeps its relative precision at any
//     magnitude.  The row sums add the bf16 weights the MFMA multiplies (two
//     per v_dot2_f32_bf16), so numerator and denominator see the same values.
//   * A planner (one workgroup of the merge launch, see planner.h) lists the
//     (sequence, row tile) items of the prefill sequences in the workspace,
//     longest first (most key tiles), so that no workgroup is launched for
//     decode rows and the longest items do not start last; workgroup ids take the KV heads fastest, so with 8 KV
//     heads each XCD runs one head's items and keeps its K/V rows in its L2.
#include "common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kWavesP = 4;
constexpr int kPairsPerWave = 32;                          // one 32-column MFMA group
constexpr int kPairsPerBlock = kWavesP * kPairsPerWave;    // 128
constexpr int kBuf = 2;                                    // K/V tiles resident in LDS
static_assert(kPairsPerBlock == kPrefillPairs, "planner and kernel agree on the row tile");
constexpr int kKT = 64;                                    // keys per tile
constexpr float kRescaleSlack = 8.f;                       // lazy max: rescale past 2^8 growth

typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4v lds_short4;
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate that waits until at most N vector-memory operations of this wave are
// outstanding (the other counters are left alone).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt immediate that waits until at most N LDS operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_lds() {
  static_assert(N >= 0 && N < 16, "lgkmcnt is four bits");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (N << 8) | (3 << 14));
}

// Two floats at an 8-byte aligned address, stored and loaded at agent scope: the store is
// written through to the level where all XCDs of the device see it, the load reads from
// there (never a stale copy in this XCD's L2).
__device__ __forceinline__ void store_coherent2(float* p, float a, float b) {
  const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_coherent2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

// Workgroup barrier for LDS hand-over: no memory operation moves across it in the
// compiler, and unlike __syncthreads() it does not wait for this wave's outstanding
// global loads (the tiles in flight).  LDS reads before it have been consumed by then.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// F8: the pools hold E4M3 codes.  Their tiles come through registers instead (16 codes
// per lane and load, widened exactly to bf16 while they are written to LDS after the
// current tile's products), the K pool scale is folded into the score scale and the V
// pool scale into the output.
template <int D, int G, bool F8>
__global__ __launch_bounds__(kWavesP * kWave, 2) void prefill_kernel(AttnParams p) {
  constexpr int CH = D / 8;                 // 16-byte bf16 chunks per K/V row in LDS
  constexpr int KS = D / 16;                // k-steps of the QK product
  constexpr int DT = D / 32;                // 32-wide dim tiles of the output
  constexpr int ROWS = kPairsPerBlock / G;  // query rows per workgroup
  constexpr int EB = F8 ? 1 : 2;            // bytes per pool value
  constexpr int CHG = D * EB / 16;          // 16-byte chunks per row in the pool
  constexpr int RW = kWave / CHG;           // rows per wave-wide load
  constexpr int RB = kWavesP * RW;          // rows per workgroup-wide load
  constexpr int NLD = kKT / RB;             // loads per thread per tile, for K and for V
  static_assert(kKT % RB == 0, "a tile is a whole number of workgroup-wide loads");

  // K and V of kBuf tiles (the one being multiplied and the ones in flight), as distinct
  // arrays: every access names its buffer at compile time (the tile loop is unrolled by
  // kBuf), so the compiler can tell a buffer being filled from one being read.
  __shared__ __attribute__((aligned(16))) uint4 k_lds0[kKT][CH], k_lds1[kKT][CH];
  __shared__ __attribute__((aligned(16))) uint4 v_lds0[kKT][CH], v_lds1[kKT][CH];
  static_assert(kBuf == 2, "two buffers declared");
  auto kbuf = [&](auto b) -> uint4 (*)[CH] {
    if constexpr (decltype(b)::value == 0) return k_lds0;
    else return k_lds1;
  };
  auto vbuf = [&](auto b) -> uint4 (*)[CH] {
    if constexpr (decltype(b)::value == 0) return v_lds0;
    else return v_lds1;
  };

  // workgroup id -> (work item, KV head), heads fastest: workgroups are handed to the 8
  // XCDs round-robin, so with 8 KV heads each XCD takes one head's items (its K/V rows
  // stay in that XCD's L2 across the row tiles of a sequence), in the planner's
  // longest-first order; items past the planner's count do nothing
  const int h = (int)(blockIdx.x % p.Hkv), item = (int)(blockIdx.x / p.Hkv);
  if (item >= *p.plan_count || item >= p.plan_capacity) return;
  const int4 it = p.plan_items[item];
  const int s = it.x, mt = it.y;
  const int piece = it.z & 0xffff, npieces = it.z >> 16;   // keys of piece `piece` of npieces
  const int slot0 = it.w;                        // first partial slot of a split item
  if (npieces < 1 || piece >= npieces) return;
  const int row0 = p.qsl[s];
  const int qn = p.qsl[s + 1] - row0;
  if (qn <= p.decode_max_q) return;              // decode rows are handled elsewhere
  const int j0 = mt * ROWS;
  if (j0 >= qn) return;
  if (row0 < 0 || row0 + qn > p.num_q_tokens) return;
  const int BS = p.bs;                           // a power of two (checked by the host)
  const int bs_shift = __builtin_ctz(BS);
  const int L = min(p.seq_lens[s], p.max_blocks * BS);   // clamp a length the table cannot map
  const int prior = L - qn;
  const int j1 = min(j0 + ROWS, qn);
  const int key_end = prior + j1;                // keys [0, key_end) are needed by this block
  if (key_end <= 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = uniform(tid / kWave);
  const int Hq = p.Hkv * G;
  const int* bt_row = p.block_tables + (size_t)s * p.max_blocks;
  const int nblocks = p.num_blocks > 0x7fffffff ? 0x7fffffff : (int)p.num_blocks;
  const uint32_t row_bytes = (uint32_t)p.Hkv * D * EB;
  const size_t blk_bytes = (size_t)BS * row_bytes;
  const char* kbase = p.k_cache + (size_t)h * D * EB;
  const char* vbase = p.v_cache + (size_t)h * D * EB;

  // ---- this lane's pair (accumulator / B-operand column n) ----
  const int n = lane & 31;
  const int kg = lane >> 5;                      // half-wave: k-group of operands, row group of results
  const int pair = w * kPairsPerWave + n;
  const int jrow = j0 + pair / G;
  const int gq = pair % G;
  const bool pvalid = jrow < j1;
  const int lim = pvalid ? prior + jrow : 0;     // last key this pair attends; invalid pairs see key 0 only
  // wave-level bounds of the causal limits (uniform)
  const int wj_lo = j0 + (w * kPairsPerWave) / G;
  const int wj_hi = j0 + (w * kPairsPerWave + kPairsPerWave - 1) / G;
  const bool wave_active = wj_lo < j1;
  const int wave_lim_min = prior + min(wj_lo, j1 - 1);
  const int wave_lim_max = prior + min(wj_hi, j1 - 1);

  // Scores enter the softmax as c s, c = scale log2(e).  The kernel works with |c| (at
  // least FLT_MIN, so masked -inf scores stay -inf): for c < 0 the query is negated,
  // which is exact in bf16, and then max(c s) = |c| max(s) and 2^(c s - m) is one fma
  // and one exp2 per score.
  const float c_in = p.scale_log2;
  const uint32_t qflip = c_in < 0.f ? 0x80008000u : 0u;
  const float c = fmaxf(fabsf(c_in), FLT_MIN);

  // ---- Q^T as the B operand: pair column n, dims ks*16 + kg*8 .. +8 ----
  bf16x8 qreg[KS];
  {
    const uint16_t* qp = p.q + ((size_t)(row0 + (pvalid ? jrow : j0)) * Hq + (size_t)h * G + gq) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (pvalid) v = *reinterpret_cast<const uint4*>(qp + ks * 16 + kg * 8);
      v.x ^= qflip; v.y ^= qflip; v.z ^= qflip; v.w ^= qflip;
      qreg[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  floatx16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  float m_run = -INFINITY, l_part = 0.f;

  // ---- tile loads: global -> LDS directly (global_load_lds_dwordx4) ----
  // Load i of wave w fills rows RB*i + RW*w .. +RW-1 of a tile: 1 KB of LDS written at
  // base + 16 * lane, so lane (row lrow, slot pc) fetches the chunk that the swizzle puts
  // there, pc ^ chunk_swizzle(row).  The rows of one load lie in one pool block (block sizes are
  // multiples of RW), so its block id is wave-uniform.  Rows at or past key_end fetch
  // row key_end - 1 instead: finite data that the causal mask gives weight 0.
  // The table entries of a tile come from one vector load (lane j: block kb / BS + j,
  // clamped to the last needed block) issued right after the previous tile's loads, so
  // the wait for that tile covers it; each load then reads its block id with readlane.
  const int lrow = lane / CHG, pc = lane % CHG;
  const int last_blk = (key_end - 1) >> bs_shift;
  auto fetch_bt = [&](int kb) -> int {
    return bt_row[min((kb >> bs_shift) + lane, last_blk)];
  };
  auto issue = [&](auto b, int kb, int btv) {
    uint4 (*kd)[CH] = kbuf(b);
    uint4 (*vd)[CH] = vbuf(b);
    uint32_t src_row[NLD];
    size_t blk_off[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int g_tok = kb + RB * i + RW * w;    // first row of load i (wave-uniform)
      const int tok = min(g_tok, key_end - 1);
      const int bl = __builtin_amdgcn_readlane(btv, (tok >> bs_shift) - (kb >> bs_shift));
      blk_off[i] = (size_t)((unsigned)bl < (unsigned)nblocks ? bl : 0) * blk_bytes;   // out-of-pool: block 0
      src_row[i] = (uint32_t)((tok & (BS - 1)) + min(lrow, max(key_end - 1 - g_tok, 0)));
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int r = RB * i + RW * w + lrow;      // tile row this lane's chunk belongs to
      const size_t off = blk_off[i] + src_row[i] * row_bytes + (uint32_t)((pc ^ chunk_swizzle<CH>(r)) * 16);
      __builtin_amdgcn_global_load_lds(kbase + off, (lds_void*)&kd[RB * i + RW * w][0], 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int r = RB * i + RW * w + lrow;
      const size_t off = blk_off[i] + src_row[i] * row_bytes + (uint32_t)((pc ^ chunk_swizzle<CH>(r)) * 16);
      __builtin_amdgcn_global_load_lds(vbase + off, (lds_void*)&vd[RB * i + RW * w][0], 16, 0, 0);
    }
  };

  // E4M3 tiles: load i of a lane brings the 16 codes of row RB i + RW w + lrow, values
  // 16 pc .. 16 pc + 15, with the same row choice and clamping as the loads above; they are
  // written as bf16 chunks 2 pc and 2 pc + 1 of that row (swizzled like every chunk).
  auto load_regs = [&](int kb, int btv, u32x4 (&kr)[NLD], u32x4 (&vr)[NLD]) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int g_tok = kb + RB * i + RW * w;
      const int tok = min(g_tok, key_end - 1);
      const int bl = __builtin_amdgcn_readlane(btv, (tok >> bs_shift) - (kb >> bs_shift));
      const size_t blk_off = (size_t)((unsigned)bl < (unsigned)nblocks ? bl : 0) * blk_bytes;
      const uint32_t src_row = (uint32_t)((tok & (BS - 1)) + min(lrow, max(key_end - 1 - g_tok, 0)));
      const size_t off = blk_off + src_row * row_bytes + (uint32_t)(pc * 16);
      kr[i] = *reinterpret_cast<const u32x4*>(kbase + off);
      vr[i] = *reinterpret_cast<const u32x4*>(vbase + off);
    }
  };
  auto store_lds = [&](auto b, const u32x4 (&kr)[NLD], const u32x4 (&vr)[NLD]) {
    uint4 (*kd)[CH] = kbuf(b);
    uint4 (*vd)[CH] = vbuf(b);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int r = RB * i + RW * w + lrow;
      const int c0 = (2 * pc) ^ chunk_swizzle<CH>(r), c1 = (2 * pc + 1) ^ chunk_swizzle<CH>(r);
      uint4 lo, hi;
      e4m3x16_to_bf16(make_uint4(kr[i].x, kr[i].y, kr[i].z, kr[i].w), lo, hi);
      kd[r][c0] = lo;
      kd[r][c1] = hi;
      e4m3x16_to_bf16(make_uint4(vr[i].x, vr[i].y, vr[i].z, vr[i].w), lo, hi);
      vd[r][c0] = lo;
      vd[r][c1] = hi;
    }
  };

  // Per-lane LDS addressing.  The A operand of the QK product for key half kh and
  // k-step ks is row 32 kh + n, chunk 2 ks + kg.  The transposing V reads of k-step kk
  // and dim tile dt: lane a of a 16-lane group points at key 16 kk + 4 kg + a / 4 (and
  // +8), dims 32 dt + dsub .. +3, so that lane i of the group receives, as its element j,
  // dim 32 dt + 16 ((lane / 16) % 2) + i of key 16 kk + 4 kg + j (and +8): the keys of the
  // B operand's elements (the score accumulator layout).
  const int a16 = lane & 15;
  const int dsub = 16 * ((lane >> 4) & 1) + 4 * (a16 & 3);

  auto tile_compute = [&](auto b, int kb) {
    uint4 (*kt)[CH] = kbuf(b);
    uint4 (*vt)[CH] = vbuf(b);

    // ---- S^T = K Q^T: 2 KS MFMAs in (ks, key half) order, operand reads kAhead ahead ----
    constexpr int NQK = 2 * KS;
    constexpr int kAhead = 6;
    auto kread = [&](auto mc) -> uint4 {
      constexpr int m = decltype(mc)::value;
      const int r = (m % 2) * 32 + n;
      return kt[r][(2 * (m / 2) + kg) ^ chunk_swizzle<CH>(r)];
    };
    uint4 kop[NQK];
    floatx16 sacc[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kh][i] = 0.f;
    static_for<kAhead>([&](auto mc) { kop[decltype(mc)::value] = kread(mc); });
    __builtin_amdgcn_sched_barrier(0);
    static_for<NQK>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      sacc[m % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kop[m]), qreg[m / 2],
                                                            sacc[m % 2], 0, 0, 0);
      if constexpr (m + kAhead < NQK) kop[m + kAhead] = kread(IntC<m + kAhead>());
      __builtin_amdgcn_sched_barrier(0);
    });

    // ---- causal mask (tiles that cross a row's diagonal only), tile max ----
    // accumulator element i of half kh holds key kb + 32 kh + 8 (i / 4) + 4 kg + i % 4
    if (kb + kKT - 1 > wave_lim_min) {
      const int rel = lim - kb - 4 * kg;         // elements at offsets above rel are masked
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * kh + 8 * (i / 4) + (i % 4) > rel) sacc[kh][i] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[kh][i]);
    {
      const int x = __float_as_int(tmax);
      const auto sw = __builtin_amdgcn_permlane32_swap(x, x, false, false);
      tmax = fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1]));
    }
    const float m_new = fmaxf(m_run, tmax * c);   // a fully masked column keeps its max

    // ---- lazy rescale: only when some row's max has grown past the slack ----
    if (__builtin_amdgcn_ballot_w64(m_new > m_run + kRescaleSlack) != 0) {
      const float alpha = fast_exp2(m_run - m_new);   // 0 on the first tile
      m_run = m_new;
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
    }

    // ---- O^T += V^T P^T over four 16-key steps; the weights of step kk + 1 are
    //      computed while the MFMAs of step kk run ----
    const float neg_m = -m_run;
    float psum = 0.f;
    auto vread = [&](int kk, int dt) -> bf16x8 {
      const int t_lo = 16 * kk + 4 * kg + (a16 >> 2);
      const int t_hi = t_lo + 8;
      const int dim = 32 * dt + dsub;
      const int ch = dim / 8, half = (dim % 8) / 4;
      const short* lo_p = reinterpret_cast<const short*>(&vt[t_lo][ch ^ chunk_swizzle<CH>(t_lo)]) + 4 * half;
      const short* hi_p = reinterpret_cast<const short*>(&vt[t_hi][ch ^ chunk_swizzle<CH>(t_hi)]) + 4 * half;
      const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)lo_p);
      const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)hi_p);
      const short8v av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return __builtin_bit_cast(bf16x8, av);
    };
    // weights 2^(c s - m) of step kk (below 2^8) as the bf16 B operand; the row sum adds
    // the same bf16 values (two per v_dot2_f32_bf16)
    auto make_p = [&](auto kkc) -> bf16x8 {
      constexpr int kk = decltype(kkc)::value;
      bf16x8 pv;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        pv[j] = (__bf16)fast_exp2(fmaf(sacc[kk >> 1][(kk & 1) * 8 + j], c, neg_m));   // 0 when masked
      const uint4 pw = __builtin_bit_cast(uint4, pv);
      psum = dot2_bf16(pw.x, 0x3f803f80u, psum);   // + p0 + p1 (a pair of bf16 ones)
      psum = dot2_bf16(pw.y, 0x3f803f80u, psum);
      psum = dot2_bf16(pw.z, 0x3f803f80u, psum);
      psum = dot2_bf16(pw.w, 0x3f803f80u, psum);
      return pv;
    };
    bf16x8 vop[2][DT];
    bf16x8 pb[4];
    static_for<DT>([&](auto dt) { vop[0][decltype(dt)::value] = vread(0, dt); });
    pb[0] = make_p(IntC<0>());
    __builtin_amdgcn_sched_barrier(0);
    static_for<4>([&](auto kkc) {
      constexpr int kk = decltype(kkc)::value;
      if constexpr (kk + 1 < 4)
        static_for<DT>([&](auto dt) { vop[(kk + 1) % 2][decltype(dt)::value] = vread(kk + 1, dt); });
      static_for<DT>([&](auto dtc) {
        constexpr int dt = decltype(dtc)::value;
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[kk % 2][dt], pb[kk], oacc[dt], 0, 0, 0);
      });
      if constexpr (kk + 1 < 4) pb[kk + 1] = make_p(IntC<kk + 1>());
      __builtin_amdgcn_sched_barrier(0);
    });
    l_part += psum;
  };

  // ---- pipeline over tiles: tile t in buffer t % kBuf, the next kBuf - 1 tiles in flight ----
  // Per thread, a tile is 2 NLD loads (K then V) issued in tile order, so "tile t has
  // landed" is "at most the loads of the tiles issued after it are outstanding".
  // A piece covers the item's key tiles [kt0, kt1): tile t of the loop is key tile kt0 + t.
  const int item_tiles = (key_end + kKT - 1) / kKT;
  // (item_tiles < 2^25 and npieces <= 32: the products fit 32 bits)
  const int kt0 = npieces == 1 ? 0 : (int)((uint32_t)(piece * item_tiles) / (uint32_t)npieces);
  const int ntiles = npieces == 1 ? item_tiles : (int)((uint32_t)((piece + 1) * item_tiles) / (uint32_t)npieces) - kt0;
  const int kb0 = kt0 * kKT;
  if constexpr (!F8) {
    int btv = fetch_bt(kb0);
    issue(IntC<0>(), kb0, btv);
    if (ntiles > 1) btv = fetch_bt(kb0 + kKT);
    auto step = [&](auto b, int t) {
      constexpr int B = decltype(b)::value;
      const int kb = kb0 + t * kKT;
      wait_vmem<0>();                            // this thread's part of tile t (and the next table entries) landed
      lds_barrier();                             // all of tile t visible; buffer (t+1) % 2 no longer read
      if (t + 1 < ntiles) {
        issue(IntC<(B + 1) % kBuf>(), kb + kKT, btv);
        if (t + 2 < ntiles) btv = fetch_bt(kb + 2 * kKT);
      }
      if (wave_active && kb <= wave_lim_max) tile_compute(b, kb);
    };
    for (int t = 0; t < ntiles; t += kBuf) {
      step(IntC<0>(), t);
      if (t + 1 < ntiles) step(IntC<1>(), t + 1);
    }
  } else {
    // E4M3: tile t + 1 is loaded into registers during step t and written to LDS after
    // tile t's products; the barrier that opens step t + 1 makes it visible.
    (void)issue;
    int btv = fetch_bt(kb0);
    {
      u32x4 kr[NLD], vr[NLD];
      load_regs(kb0, btv, kr, vr);
      store_lds(IntC<0>(), kr, vr);
    }
    if (ntiles > 1) btv = fetch_bt(kb0 + kKT);
    auto step = [&](auto b, int t) {
      constexpr int B = decltype(b)::value;
      const int kb = kb0 + t * kKT;
      wait_lds<0>();                             // this wave's writes of tile t are done
      lds_barrier();                             // all of tile t visible; buffer (t+1) % 2 no longer read
      const bool more = t + 1 < ntiles;
      u32x4 kr[NLD], vr[NLD];
      if (more) load_regs(kb + kKT, btv, kr, vr);
      if (t + 2 < ntiles) btv = fetch_bt(kb + 2 * kKT);
      if (wave_active && kb <= wave_lim_max) tile_compute(b, kb);
      if (more) store_lds(IntC<(B + 1) % kBuf>(), kr, vr);
    };
    for (int t = 0; t < ntiles; t += kBuf) {
      step(IntC<0>(), t);
      if (t + 1 < ntiles) step(IntC<1>(), t + 1);
    }
  }

  // ---- finish: O / l, bf16 out; lane holds dims 32 dt + 8 q + 4 kg + 0..3 of its pair ----
  const int x = __float_as_int(l_part);
  const auto sw = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  float l_tot = __int_as_float(sw[0]) + __int_as_float(sw[1]);
  if (npieces > 1) {
    // A piece of a split item: its partial (O against m_run, m_run, l) goes to the workspace
    // rows of slot slot0 + piece, KV head h, written through to the device-coherent level
    // (agent-scope stores), and the item's counter of this head is raised once they have
    // landed.  The workgroup that raises it last reads every piece's partial the same way
    // and writes O = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j, M = max_j m_j (the same
    // rescale identity as the decode merge).  Every piece has at least 31 tiles and the last
    // one starts below the item's first row, so every valid pair sees keys in every piece.
    auto row_of = [&](int j) -> int64_t {
      return ((int64_t)(slot0 + j) * p.Hkv + h) * kPrefillPairs + pair;
    };
    if (pvalid) {
      float* po = p.ws_o + row_of(piece) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = dt * 32 + 8 * q4 + 4 * kg;
          store_coherent2(po + d, oacc[dt][q4 * 4 + 0], oacc[dt][q4 * 4 + 1]);
          store_coherent2(po + d + 2, oacc[dt][q4 * 4 + 2], oacc[dt][q4 * 4 + 3]);
        }
      if (kg == 0) {
        __hip_atomic_store(p.ws_m + row_of(piece), m_run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.ws_l + row_of(piece), l_tot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    wait_vmem<0>();                              // this thread's partial has landed
    __syncthreads();
    __shared__ int last_piece;
    if (threadIdx.x == 0)
      last_piece = __hip_atomic_fetch_add(p.plan_split_ctr + (size_t)slot0 * p.Hkv + h, 1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == npieces - 1;
    __syncthreads();
    if (!last_piece || !pvalid) return;
    float M = -INFINITY;
    for (int j = 0; j < npieces; ++j)
      M = fmaxf(M, __hip_atomic_load(p.ws_m + row_of(j), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
    l_tot = 0.f;
    for (int j = 0; j < npieces; ++j) {
      const float mj = __hip_atomic_load(p.ws_m + row_of(j), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float wj = fast_exp2(mj - M);
      l_tot += wj * __hip_atomic_load(p.ws_l + row_of(j), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float* po = p.ws_o + row_of(j) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = dt * 32 + 8 * q4 + 4 * kg;
          const float2 a = load_coherent2(po + d), b2 = load_coherent2(po + d + 2);
          oacc[dt][q4 * 4 + 0] += wj * a.x;
          oacc[dt][q4 * 4 + 1] += wj * a.y;
          oacc[dt][q4 * 4 + 2] += wj * b2.x;
          oacc[dt][q4 * 4 + 3] += wj * b2.y;
        }
    }
  }
  if (!pvalid) return;
  const float inv = F8 ? p.v_scale / l_tot : 1.f / l_tot;
  uint16_t* op = p.out + ((size_t)(row0 + jrow) * Hq + (size_t)h * G + gq) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = dt * 32 + 8 * q4 + 4 * kg;
      const uint32_t w0 = pack_bf16x2(oacc[dt][q4 * 4 + 0] * inv, oacc[dt][q4 * 4 + 1] * inv);
      const uint32_t w1 = pack_bf16x2(oacc[dt][q4 * 4 + 2] * inv, oacc[dt][q4 * 4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + d) = make_uint2(w0, w1);
    }
}

template <int D, bool F8>
hipError_t dispatch_g(const AttnParams& p, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  // the work list was written by the planner workgroup of the merge launch; one workgroup
  // per (possible item, KV head)
  dim3 grid((unsigned)((int64_t)p.Hkv * p.plan_stride));
  switch (G) {
    case 1: hipLaunchKernelGGL((prefill_kernel<D, 1, F8>), grid, dim3(kWavesP * kWave), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<D, 2, F8>), grid, dim3(kWavesP * kWave), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<D, 4, F8>), grid, dim3(kWavesP * kWave), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<D, 8, F8>), grid, dim3(kWavesP * kWave), 0, stream, p); break;
    case 16: hipLaunchKernelGGL((prefill_kernel<D, 16, F8>), grid, dim3(kWavesP * kWave), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool prefill_supported(int D, int G, int bs, bool fp8) {
  // a wave-wide tile load (64 / (16-byte chunks per pool row) rows) must stay inside one
  // pool block, and a tile (64 keys) must hold whole blocks
  const int chunks = D * (fp8 ? 1 : 2) / 16;
  return (D == 64 || D == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16) &&
         (bs == 8 || bs == 16 || bs == 32) && bs % (kWave / chunks) == 0;
}

hipError_t launch_prefill(const AttnParams& p, bool fp8, hipStream_t stream) {
  if (p.max_query_len <= p.decode_max_q) return hipSuccess;   // decode rows only
  if (fp8) {
    if (p.D == 128) return dispatch_g<128, true>(p, stream);
    if (p.D == 64) return dispatch_g<64, true>(p, stream);
  } else {
    if (p.D == 128) return dispatch_g<128, false>(p, stream);
    if (p.D == 64) return dispatch_g<64, false>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
