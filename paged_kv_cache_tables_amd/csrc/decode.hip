// Decode rows (one query token per sequence, or a few for short chunks such as
// speculative verification): split-K paged attention plus a log-sum-exp merge of
// the pieces.
//
// What is computed is the exact softmax attention of "Under the Hood: Flash
// Attention" (Text Generation Inference page): a running max m, a running sum
// l of exponentials and an output accumulator rescaled by exp(m_old - m_new)
// whenever the max grows, finished by O / l.  The same rescale identity
// merges partial (O, m, l) triples computed over disjoint key ranges, which is
// what the merge kernel does across pieces.  Keys and values are reached
// through the sequence's block table ("Under the Hood: PagedAttention").
//
// Why matrix cores for a bandwidth-bound step: with a GQA group of G query
// heads sharing each K/V row, decode performs G floating-point operations per
// byte of K/V (G*D multiply-adds for QK and again for PV per 4*D bytes).  At
// 8 TB/s and G = 8 that is 64 TFLOP/s of fp32 FMAs -- 81% of the chip's
// non-packed fp32 vector peak before any softmax work -- so vector-ALU decode
// would be ALU-bound below the HBM roofline.  The group's products are real
// dense contractions ([G x D] x [D x T]), so they run on bf16 MFMA with fp32
// accumulation and the vector ALUs are left with the softmax.
//
// Layout (gfx950, v_mfma_f32_16x16x32_bf16):
//   * Partition: the decode rows' work is cut into units (sequence, group of
//     KV heads, 64-token tile), in that order.  The grid has one wave per
//     resident wave slot of the device; a workgroup holds one wave per KV head
//     of a group (up to 8) and takes an equal consecutive share of units,
//     walked as pieces of consecutive (sequence, group) segments.  The waves
//     of a workgroup read the same slots for different heads, and a slot's
//     heads sit side by side in the pool, so the DRAM rows behind each slot
//     are read together.
//   * Loads are fully coalesced: 16 lanes read one 256-byte row (16 bytes each),
//     4 rows per instruction; the pool block of each instruction is
//     wave-uniform (scalar base).  K and V of a tile arrive in registers.
//   * Both tiles pass through one per-wave LDS buffer, row-major with a XOR
//     swizzle of the 16-byte chunks (row r's chunk c sits at c ^ (r % CH)):
//     first K, read back as MFMA A operands (16 contiguous bytes per lane,
//     conflict-free), then V, read back transposed with ds_read_b64_tr_b16.
//   * Scores transposed, S^T = K Q^T: A = 16 key rows x 32 dims, B = the G
//     query rows (heads padded to 16 columns, loaded once).  Each lane's
//     accumulator column is one head: the per-head max and sum need a local
//     reduction plus two lane exchanges.
//   * Output transposed, O^T = V^T P^T: B = P^T is the score accumulator
//     rounded to bf16 in place (the row sum adds the same rounded weights); A = V^T.
//   * Streaming: each register set is refilled with the next tile as soon as
//     its contents are in LDS, so K and V both run one tile ahead.
//   * Fused append: positions that are this call's new tokens are read from the
//     new rows (k_new / v_new) instead of the pools, which the merge launch
//     fills afterwards.
//   A piece that covers its whole (sequence, head) writes bf16 output directly;
//   otherwise fp32 partials (O, m, l) go to the workspace for the merge kernel.
#include <algorithm>
#include <climits>

#include "common.h"
#include "kernels.h"
#include "planner.h"

namespace pkv {

namespace {

constexpr int kTile = 64;        // tokens per tile

typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4v lds_short4;

// First query row, row count, key count and 64-token tiles of sequence s when its rows
// are decode rows -- 1 <= q_s <= decode_max_q, so that its q_s x G (row, head) columns fit
// the 16 columns of the score product -- and no tiles otherwise.
struct SeqInfo {
  int row0, q, len, tiles;
};
__device__ __forceinline__ SeqInfo seq_info(const AttnParams& p, int s) {
  const int row0 = p.qsl[s];
  const int q = p.qsl[s + 1] - row0;
  const int len = min(p.seq_lens[s], p.max_blocks * p.bs);   // clamp a length the table cannot map
  if (q < 1 || q > p.decode_max_q || row0 < 0 || row0 + q > p.num_q_tokens || len <= 0)
    return SeqInfo{row0, 0, 0, 0};
  return SeqInfo{row0, q, len, (len + kTile - 1) / kTile};
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d *= 2) {
    const int y = __shfl_up(v, d, kWave);
    if (lane >= d) v += y;
  }
  return v;
}

// MULTI: some sequence may have several decode rows (decode_max_q > 1); otherwise every
// column's causal limit is the sequence's last key and only the tile end masks.
// F8: the pools hold E4M3 codes (one byte per value); rows are widened to bf16 (exactly:
// every E4M3 value is a bf16 value) on their way into LDS, the K pool scale is folded
// into the score scale and the V pool scale into the output.
template <int D, int G, int BS, bool MULTI, bool F8>
__global__ __launch_bounds__(kMaxDecodeGroup * kWave) __attribute__((amdgpu_waves_per_eu(2, 8)))
void decode_kernel(AttnParams p) {
  constexpr int CH = D / 8;              // 16-byte bf16 chunks per row in LDS
  constexpr int EB = F8 ? 1 : 2;         // bytes per pool value
  constexpr int CHG = D * EB / 16;       // 16-byte chunks per row in the pool
  constexpr int RPI = kWave / CHG;       // rows per wave-wide load (4 at d 128, 8 for E4M3)
  constexpr int NL = kTile / RPI;        // loads per lane per tile, for K and for V
  constexpr int KS = D / 32;             // k-steps of QK (32 dims each)
  constexpr int DB = D / 16;             // 16-dim blocks of the output
  constexpr int TB = kTile / 16;         // 16-token blocks of a tile
  constexpr int NBT = kTile / BS;        // pool blocks spanned by a tile
  static_assert(G <= 16, "a GQA group is one 16-column MFMA tile");
  static_assert(kTile % BS == 0 && BS % RPI == 0, "a wave-wide load stays inside one pool block");

  // one [kTile][CH] tile per wave: K, then V, of the wave's current tile
  extern __shared__ __attribute__((aligned(16))) uint4 lds_tiles[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = uniform((int)(threadIdx.x / kWave));   // wave of the workgroup = KV head within the group
  uint4 (*tile)[CH] = reinterpret_cast<uint4 (*)[CH]>(lds_tiles + (size_t)wv * kTile * CH);
  const int w = blockIdx.x;                      // workgroup = one share of the units
  const int Hkv = p.Hkv;
  const int WPG = p.decode_group;                // KV heads (waves) per workgroup; divides Hkv
  const int NG = Hkv / WPG;                      // head groups

  // ---- the partition: units (s, head group, tile) in that order, an equal share per workgroup ----
  // The waves of a workgroup take the same units for the heads of one group, so the heads'
  // rows of each pool slot (adjacent in memory) are read at the same time.  Lane l sums the
  // tiles of sequences [l c, (l + 1) c); a wave scan gives each lane the units before its
  // chunk.  Unit counts fit in 32 bits (checked by the host).
  const int c_per = (p.num_seqs + kWave - 1) / kWave;
  int my_tiles = 0;
  SeqInfo first{0, 0, 0, 0};                     // this lane's first sequence
  for (int i = 0; i < c_per; ++i) {
    const int s = lane * c_per + i;
    if (s < p.num_seqs) {
      const SeqInfo si = seq_info(p, s);
      if (i == 0) first = si;
      my_tiles += si.tiles;
    }
  }
  const int incl = wave_incl_scan(my_tiles);
  const int total_units = uniform(__shfl(incl, kWave - 1, kWave) * NG);
  if (total_units == 0) return;
  const int nwg = p.decode_waves / WPG;          // workgroups of the grid
  const int share = uniform(max(p.min_share_tiles, (total_units + nwg - 1) / nwg));
  if (w >= (total_units + share - 1) / share) return;   // fewer shares than workgroups
  const int x0 = w * share;
  const int x1 = min(x0 + share, total_units);
  // the lane whose chunk holds unit x0, then the sequence inside that chunk
  const int excl_units = (incl - my_tiles) * NG;
  const unsigned long long hit = __builtin_amdgcn_ballot_w64(excl_units <= x0 && x0 < incl * NG);
  const int src = (int)__builtin_ctzll(hit);     // nonempty: x0 < total_units
  int s = uniform(src * c_per);
  int seg_a = uniform(__shfl(excl_units, src, kWave));   // first unit of sequence s
  int cur_row0 = uniform(__shfl(first.row0, src, kWave));
  int cur_q = uniform(__shfl(first.q, src, kWave));
  int cur_len = uniform(__shfl(first.len, src, kWave));
  int nt = uniform(__shfl(first.tiles, src, kWave));
  auto next_seq = [&]() {
    seg_a += NG * nt;
    s = uniform(s + 1);
    const SeqInfo si = seq_info(p, s);
    cur_row0 = uniform(si.row0);
    cur_q = uniform(si.q);
    cur_len = uniform(si.len);
    nt = uniform(si.tiles);
  };
  while (x0 >= seg_a + NG * nt && s + 1 < p.num_seqs) next_seq();

  const int n = lane & 15;                       // accumulator column: query head of the group
  const int kg = lane >> 4;                      // k-group / accumulator row group
  const int Hq = Hkv * G;
  const size_t row_stride = (size_t)Hkv * D;     // values per pool slot
  const int nblocks = p.num_blocks > 0x7fffffff ? 0x7fffffff : (int)p.num_blocks;
  const size_t blk_bytes = (size_t)BS * row_stride * EB;
  const uint32_t row_bytes = (uint32_t)(row_stride * EB);
  const float c = p.scale_log2;
  const int lrow = lane / CHG, lch = lane % CHG; // this lane's row (within a load) and chunk
  const uint32_t lane_off = (uint32_t)lrow * row_bytes + (uint32_t)lch * 16;

  // One piece: tiles [tb0, tb1) of (sequence s, KV head h), whose units start at unit a.
  auto piece = [&](int h, int tb0, int tb1, int a) {
    const int row0 = cur_row0;
    const int L = cur_len;
    // accumulator column n = (row rr of the sequence's q_s rows, head g of the group); the
    // row at position L - q_s + rr attends keys 0..lim
    const int rr = n / G, g = n % G;
    const bool col_valid = rr < cur_q;
    const int lim = col_valid ? L - cur_q + rr : L - 1;
    const int t_begin = tb0 * kTile;
    const int t_end = min(tb1 * kTile, L);
    const int* bt_row = p.block_tables + (size_t)s * p.max_blocks;
    const char* kbase = p.k_cache + (size_t)h * D * EB;
    const char* vbase = p.v_cache + (size_t)h * D * EB;
    // positions fresh0 .. L - 1 are this step's tokens; with a fused append they are not in
    // the pools yet and come from the rows of k_new / v_new instead
    const int fresh0 = (!F8 && p.k_new != nullptr) ? L - cur_q : INT_MAX;
    const uint16_t* knew_h = p.k_new + (size_t)h * D;
    const uint16_t* vnew_h = p.v_new + (size_t)h * D;

    // ---- Q^T as the B operand: column n, dims ks*32 + kg*8 .. +8 (zero for padding columns) ----
    bf16x8 qreg[KS];
    {
      const uint16_t* qp = p.q + ((size_t)(row0 + (col_valid ? rr : 0)) * Hq + (size_t)h * G + g) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (col_valid) v = *reinterpret_cast<const uint4*>(qp + ks * 32 + kg * 8);
        qreg[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }

    floatx4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_part = 0.f;

    // Block-table entries of a tile (wave-uniform scalar loads).  Entries past the end,
    // or outside the pool, become block 0: a safe address whose rows the masks ignore.
    auto load_bts = [&](int t0, int* dst) {
#pragma unroll
      for (int j = 0; j < NBT; ++j) {
        const int b = (t0 + j * BS < t_end) ? bt_row[uniform((t0 + j * BS) / BS)] : 0;
        dst[j] = (unsigned)b < (unsigned)nblocks ? b : 0;
      }
    };
    // Coalesced tile load: load i covers rows RPI*i .. RPI*i + RPI - 1 (one pool block).  A
    // tile that holds fresh positions takes those rows from the new rows instead (lane by lane).
    auto issue = [&](const char* base, const uint16_t* nbase, const int* bb, uint4* reg, int t0) {
      if (t0 + kTile > fresh0) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const char* b = base + (size_t)bb[(RPI * i) / BS] * blk_bytes + (uint32_t)((RPI * i) % BS) * row_bytes;
          const int t = t0 + RPI * i + lrow;
          const char* src = b + lane_off;
          if (t >= fresh0 && t < L)
            src = reinterpret_cast<const char*>(nbase + (size_t)(row0 + t - fresh0) * row_stride) + lch * 16;
          reg[i] = load_stream16(src);
        }
        return;
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const char* b = base + (size_t)bb[(RPI * i) / BS] * blk_bytes + (uint32_t)((RPI * i) % BS) * row_bytes;
        reg[i] = load_stream16(b + lane_off);
      }
    };
    // Registers -> LDS, row-major bf16, chunk c of row r at c ^ (r % CH); rows >= nvalid get
    // zeros.  An E4M3 lane holds 16 codes of its row, which become bf16 chunks 2 lch, 2 lch + 1.
    auto stage = [&](const uint4* reg, int nvalid) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int r = RPI * i + lrow;
        uint4 v = reg[i];
        if (nvalid < kTile && r >= nvalid) v = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (F8) {
          uint4 lo, hi;
          e4m3x16_to_bf16(v, lo, hi);
          tile[r][(2 * lch) ^ (r % CH)] = lo;
          tile[r][(2 * lch + 1) ^ (r % CH)] = hi;
        } else {
          tile[r][lch ^ (r % CH)] = v;
        }
      }
    };

    const int ntiles = (t_end - t_begin + kTile - 1) / kTile;
    // One tile: its K and V wait in kr / vr; as soon as each is in LDS the registers are
    // refilled with tile tile_i + AHEAD, so AHEAD register sets keep AHEAD tiles in flight.
    auto tile_step = [&](uint4* kr, uint4* vr, int tile_i, auto ahead_c) {
      constexpr int AHEAD = decltype(ahead_c)::value;
      const int ts = t_begin + tile_i * kTile;
      const int nvalid = min(kTile, t_end - ts);
      const bool refill = tile_i + AHEAD < ntiles;
      const int tn = ts + AHEAD * kTile;
      int bts_n[NBT];
#pragma unroll
      for (int j = 0; j < NBT; ++j) bts_n[j] = 0;
      if (refill) load_bts(tn, bts_n);

      // ---- K tile -> LDS; refill the K registers with tile tile_i + AHEAD ----
      stage(kr, nvalid);
      __builtin_amdgcn_sched_barrier(0);
      if (refill) issue(kbase, knew_h, bts_n, kr, tn);
      wave_lds_sync();

      // ---- S^T = K Q^T ----
      floatx4 sacc[TB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        sacc[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
        const int r = tb * 16 + n;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 kv = tile[r][(ks * 4 + kg) ^ (r % CH)];
          sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv), qreg[ks], sacc[tb], 0, 0, 0);
        }
      }
      wave_lds_sync();                           // K reads done before V overwrites the buffer

      // ---- V tile -> LDS; refill the V registers with tile tile_i + AHEAD ----
      stage(vr, nvalid);
      __builtin_amdgcn_sched_barrier(0);
      if (refill) issue(vbase, vnew_h, bts_n, vr, tn);

      // ---- online softmax for column n over this tile's tokens (exp2 domain) ----
      const int last = MULTI ? min(nvalid - 1, lim - ts) : nvalid - 1;   // last token column n sees
      float tmax = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = tb * 16 + 4 * kg + i;    // token of this accumulator element
          const float v = (r <= last) ? sacc[tb][i] * c : -INFINITY;
          sacc[tb][i] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
      const float mn = fmaxf(m_run, tmax);       // -inf while column n has seen no key of this piece
      // a column that has seen no key of this piece (only with several rows) keeps weights 0
      const float m_use = (MULTI && mn == -INFINITY) ? 0.f : mn;
      const float alpha = fast_exp2(m_run - m_use);   // 0 until the column's first visible key
      m_run = mn;
      // the weights are rounded to bf16 here, once: the row sum adds exactly the values the
      // PV product multiplies, so numerator and denominator see the same weights
      float psum = 0.f;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = round_bf16(fast_exp2(sacc[tb][i] - m_use));   // 0 for masked tokens
          sacc[tb][i] = e;
          psum += e;
        }
      l_part = l_part * alpha + psum;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[db][i] *= alpha;
      wave_lds_sync();                           // V is in LDS

      // ---- O^T += V^T P^T, two 32-token k-steps ----
      // The A operand of lane (dim n, k-group kg) holds tokens t_lo + 0..3 and t_lo + 16..19
      // (t_lo = 32 kk + 4 kg), matching the score accumulator layout of the B operand.  A
      // transposing read returns, in lane i of a 16-lane group, element i % 4 of the 8 bytes
      // addressed by lane 4 j + i / 4 as its element j: lane a of the group therefore points
      // at token t_lo + a / 4, dims d0 + 4 (a % 4) .. +3.
#pragma unroll
      for (int kk = 0; kk < TB / 2; ++kk) {
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[i] = (__bf16)sacc[2 * kk][i];
          pb[4 + i] = (__bf16)sacc[2 * kk + 1][i];
        }
        const int tr = 32 * kk + 4 * kg + n / 4; // token row this lane addresses
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int dim = db * 16 + 4 * (n % 4); // first of the 4 dims this lane addresses
          const int ch = dim / 8, half = (dim % 8) / 4;
          const short* lo_p = reinterpret_cast<const short*>(&tile[tr][ch ^ (tr % CH)]) + 4 * half;
          const short* hi_p = reinterpret_cast<const short*>(&tile[tr + 16][ch ^ ((tr + 16) % CH)]) + 4 * half;
          const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)lo_p);
          const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)hi_p);
          const short8v av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), pb, oacc[db], 0, 0, 0);
        }
      }
      wave_lds_sync();                           // V reads done before the next K lands
    };
    int bts[NBT];
    load_bts(t_begin, bts);
    // one register set: K and V run one tile ahead (for 8-bit pools a second set, two tiles
    // ahead, measured slower: 69 -> 79 us per call on the Llama-3-8B batch)
    uint4 kreg[NL], vreg[NL];
    issue(kbase, knew_h, bts, kreg, t_begin);
    issue(vbase, vnew_h, bts, vreg, t_begin);
    for (int tile_i = 0; tile_i < ntiles; ++tile_i) tile_step(kreg, vreg, tile_i, IntC<1>());

    // ---- finish: lane (kg, n) holds dims db*16 + 4kg + i of column n ----
    // (the column's row and head are recomputed here rather than kept live through the loop)
    int n_e = n, kg_e = kg;
    asm volatile("" : "+v"(n_e), "+v"(kg_e));
    const int rr_e = n_e / G, g_e = n_e % G;
    const int first_w = a / share;                 // the workgroup holding tile 0 of (s, h)
    const int nseg = (a + nt - 1) / share - first_w + 1;   // pieces of (s, h)
    // partial slot: 2 w for the piece that opens this workgroup's share, 2 w + 1 for a later one
    // (only the last piece of a share can be a later partial one)
    const int slot = 2 * w + (a + tb0 != x0 ? 1 : 0);
    if (tb0 == 0 && lane == 0) p.ws_nparts[(size_t)s * Hkv + h] = make_int2(slot, nseg);
    float l_tot = l_part + __shfl_xor(l_part, 16, kWave);
    l_tot += __shfl_xor(l_tot, 32, kWave);
    if (rr_e < cur_q) {
      const int qh = h * G + g_e;
      if (nseg == 1) {                           // the whole (s, h): final output
        const float inv = F8 ? p.v_scale / l_tot : 1.f / l_tot;
        uint16_t* op = p.out + ((size_t)(row0 + rr_e) * Hq + qh) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint32_t w0 = (uint32_t)f32_to_bf16_rne(oacc[db][0] * inv) | ((uint32_t)f32_to_bf16_rne(oacc[db][1] * inv) << 16);
          const uint32_t w1 = (uint32_t)f32_to_bf16_rne(oacc[db][2] * inv) | ((uint32_t)f32_to_bf16_rne(oacc[db][3] * inv) << 16);
          *reinterpret_cast<uint2*>(op + db * 16 + 4 * kg_e) = make_uint2(w0, w1);
        }
      } else {                                   // a partial: row (slot, wave, column) of the workspace
        const size_t idx = ((size_t)slot * WPG + wv) * 16 + n_e;
        const float vs = F8 ? p.v_scale : 1.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          *reinterpret_cast<float4*>(p.ws_o + idx * D + db * 16 + 4 * kg_e) =
              make_float4(oacc[db][0] * vs, oacc[db][1] * vs, oacc[db][2] * vs, oacc[db][3] * vs);
        if (kg_e == 0) { p.ws_m[idx] = m_run; p.ws_l[idx] = l_tot; }
      }
    }
  };

  // ---- walk the share: pieces of consecutive (s, head group) segments; this wave takes
  // the head wv of each group ----
  int pos = x0;
  while (pos < x1) {
    if (pos >= seg_a + NG * nt) {                // past sequence s: next sequence with decode tiles
      if (s + 1 >= p.num_seqs) break;            // not reached: pos < total_units
      next_seq();
      continue;
    }
    const int hg = (pos - seg_a) / nt;
    const int a = seg_a + hg * nt;               // first unit of (s, hg)
    const int tb0 = pos - a;
    const int tb1 = min(x1, a + nt) - a;
    piece(hg * WPG + wv, tb0, tb1, a);
    pos = a + tb1;
  }
}

// Log-sum-exp merge of the pieces of one (decode sequence, query head):
// out = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j with M = max_j m_j.
// A piece row of D floats is D / 4 lanes of float4, so a wave reads 64 / (D / 4) pieces
// at once and adds its lane groups with lane exchanges.  Narrow form: one wave per
// (sequence, query head), four per workgroup, for calls whose segments have few pieces;
// one pass with a running max, several steps of loads in flight.
// Wide form: the four waves of a workgroup share one (sequence, query head) and are
// combined through LDS, for long sequences cut into many pieces.
constexpr int kMergeWaves = 4;

template <int D, bool WIDE>
__global__ __launch_bounds__(kMergeWaves * kWave) void merge_kernel(AttnParams p) {
  constexpr int LPP = D / 4;                     // lanes per piece row
  constexpr int PPI = kWave / LPP;               // pieces per wave-wide step
  constexpr int WPC = WIDE ? kMergeWaves : 1;    // waves per (sequence, query head)
  __shared__ float4 part[WIDE ? kMergeWaves : 1][LPP];
  __shared__ float lpart[WIDE ? kMergeWaves : 1];
  // workgroups: [planner] merge cells ... [fused append ...]
  int bid = (int)blockIdx.x;
  if (p.plan_first) {
    if (bid == 0) {                              // the prefill kernel's work list, before it runs
      __shared__ int plan_bins[kPlanBins];
      __shared__ int plan_wave_tot[kMergeWaves];
      plan_prefill_items<kMergeWaves * kWave>(p, plan_bins, plan_wave_tot);
      return;
    }
    bid -= 1;
  }
  if (bid >= p.merge_blocks) {                   // fused append: scatter the new rows into the pools
    // one thread per 16-byte chunk of a K or V row, grid-stride over the append workgroups
    const int row_chunks = p.Hkv * D / 8;
    const int64_t per_token = 2 * (int64_t)row_chunks;
    const int64_t total = p.num_q_tokens * per_token;
    const int64_t nthreads = (int64_t)(gridDim.x - p.plan_first - p.merge_blocks) * blockDim.x;
    const int64_t num_slots = p.num_blocks * p.bs;
    for (int64_t idx = (int64_t)(bid - p.merge_blocks) * blockDim.x + threadIdx.x; idx < total;
         idx += nthreads) {
      const int64_t i = idx / per_token;
      const int rem = (int)(idx - i * per_token);
      const int which = rem >= row_chunks;       // 0 = K, 1 = V
      const int c = rem - which * row_chunks;
      const int64_t slot = p.slots[i];
      if (slot < 0 || slot >= num_slots) continue;   // padding row, or outside the pool
      const uint4* src = reinterpret_cast<const uint4*>(which ? p.v_new : p.k_new);
      uint4* dst = which ? p.v_pool : p.k_pool;
      dst[slot * row_chunks + c] = src[i * row_chunks + c];
    }
    return;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = (int)(threadIdx.x / kWave);
  // cell = (sequence s, query head qh); its decode rows are merged one after the other
  const int cell = WIDE ? bid : bid * kMergeWaves + wv;
  if (cell >= p.num_seqs * p.Hq) return;         // uniform over the workgroup in the wide form
  const int s = cell / p.Hq, qh = cell % p.Hq;
  const int sub = lane / LPP, dq = lane % LPP;
  // the cell's KV head h, its wave in the decode workgroup and its column g of the group
  const int G = p.Hq / p.Hkv, h = qh / G, g = qh % G, wv_h = h % p.decode_group;
  // (the piece record is loaded together with the lengths; it is used only for sequences with
  // decode rows, whose records the decode kernel wrote)
  const int2 np = p.ws_nparts[(size_t)s * p.Hkv + h];
  const SeqInfo si = seq_info(p, s);
  const int nsplit = np.y;
  // first row of piece j's 16-column block for each wave: piece 0 in slot np.x, piece j > 0 in
  // slot 0 of the j-th following workgroup
  auto piece_row = [&](int j) -> size_t {
    const int slot = j == 0 ? np.x : 2 * (np.x / 2 + j);
    return (size_t)slot * p.decode_group * 16;
  };
  if constexpr (!WIDE) {
    // One pass with a running max, CK wave-wide steps (PPI pieces each) of loads in flight
    // at a time; lanes past the piece count load nothing and are discarded by selection,
    // never by a zero weight.
    constexpr int CK = 4;
    auto merge_row = [&](int rr, int nsplit, int row0) {
      const size_t col = (size_t)wv_h * 16 + rr * G + g;   // (wave, column) of this row's head
      float M = -INFINITY, ls = 0.f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int j0 = 0; j0 < nsplit; j0 += CK * PPI) {
        float4 o[CK];
        float mj[CK], lj[CK];
#pragma unroll
        for (int c = 0; c < CK; ++c) {
          const int j = j0 + c * PPI + sub;
          mj[c] = -INFINITY;
          lj[c] = 0.f;
          o[c] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (j < nsplit) {                      // only the pieces that exist are read
            const size_t r = piece_row(j) + col;
            mj[c] = p.ws_m[r];
            lj[c] = p.ws_l[r];
            o[c] = *reinterpret_cast<const float4*>(p.ws_o + r * D + 4 * dq);
          }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < CK; ++c)
          if (j0 + c * PPI + sub < nsplit) mx = fmaxf(mx, mj[c]);
#pragma unroll
        for (int off = LPP; off < kWave; off *= 2) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
        const float Mn = fmaxf(M, mx);           // finite: piece 0 holds key 0, seen by every row
        const float r = fast_exp2(M - Mn);       // 0 on the first round
        M = Mn;
        ls *= r;
        acc.x *= r; acc.y *= r; acc.z *= r; acc.w *= r;
#pragma unroll
        for (int c = 0; c < CK; ++c) {
          if (j0 + c * PPI + sub < nsplit) {
            const float f = fast_exp2(mj[c] - M);   // 0 for a piece that saw no key of this row
            acc.x = fmaf(f, o[c].x, acc.x); acc.y = fmaf(f, o[c].y, acc.y);
            acc.z = fmaf(f, o[c].z, acc.z); acc.w = fmaf(f, o[c].w, acc.w);
            ls = fmaf(f, lj[c], ls);
          }
        }
      }
#pragma unroll
      for (int off = LPP; off < kWave; off *= 2) {
        acc.x += __shfl_xor(acc.x, off, kWave); acc.y += __shfl_xor(acc.y, off, kWave);
        acc.z += __shfl_xor(acc.z, off, kWave); acc.w += __shfl_xor(acc.w, off, kWave);
        ls += __shfl_xor(ls, off, kWave);
      }
      if (sub == 0) {
        const float inv = 1.f / ls;
        const uint32_t w0 = (uint32_t)f32_to_bf16_rne(acc.x * inv) | ((uint32_t)f32_to_bf16_rne(acc.y * inv) << 16);
        const uint32_t w1 = (uint32_t)f32_to_bf16_rne(acc.z * inv) | ((uint32_t)f32_to_bf16_rne(acc.w * inv) << 16);
        *reinterpret_cast<uint2*>(p.out + ((size_t)(row0 + rr) * p.Hq + qh) * D + 4 * dq) = make_uint2(w0, w1);
      }
    };
    if (si.tiles == 0 || nsplit <= 1) return;    // no decode rows, or written by the decode kernel
    for (int rr = 0; rr < si.q; ++rr) merge_row(rr, nsplit, si.row0);
    return;
  }
  if (si.tiles == 0 || nsplit <= 1) return;      // no decode rows, or written by the decode kernel
  const int w_in = WIDE ? wv : 0;

  for (int rr = 0; rr < si.q; ++rr) {
    const size_t col = (size_t)wv_h * 16 + rr * G + g;
    float M = -INFINITY;                         // every wave of the cell finds the same M
    for (int j = lane; j < nsplit; j += kWave) M = fmaxf(M, p.ws_m[piece_row(j) + col]);
    M = wave_max(M);

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float ls = 0.f;
#pragma unroll 4
    for (int j = w_in * PPI + sub; j < nsplit; j += WPC * PPI) {
      const size_t r = piece_row(j) + col;
      const float f = fast_exp2(p.ws_m[r] - M);   // 0 for a piece that saw no key of this row
      const float4 o = *reinterpret_cast<const float4*>(p.ws_o + r * D + 4 * dq);
      acc.x = fmaf(f, o.x, acc.x); acc.y = fmaf(f, o.y, acc.y);
      acc.z = fmaf(f, o.z, acc.z); acc.w = fmaf(f, o.w, acc.w);
      ls = fmaf(f, p.ws_l[r], ls);
    }
#pragma unroll
    for (int off = LPP; off < kWave; off *= 2) {
      acc.x += __shfl_xor(acc.x, off, kWave); acc.y += __shfl_xor(acc.y, off, kWave);
      acc.z += __shfl_xor(acc.z, off, kWave); acc.w += __shfl_xor(acc.w, off, kWave);
      ls += __shfl_xor(ls, off, kWave);
    }
    if constexpr (WIDE) {
      if (sub == 0) part[wv][dq] = acc;
      if (lane == 0) lpart[wv] = ls;
      __syncthreads();
      for (int i = 1; i < kMergeWaves; ++i) {
        const float4 q4 = part[i][dq];
        acc.x += q4.x; acc.y += q4.y; acc.z += q4.z; acc.w += q4.w;
        ls += lpart[i];
      }
      __syncthreads();                           // LDS free for the next row
    }
    if (sub == 0 && w_in == 0) {
      const float inv = 1.f / ls;
      const uint32_t w0 = (uint32_t)f32_to_bf16_rne(acc.x * inv) | ((uint32_t)f32_to_bf16_rne(acc.y * inv) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16_rne(acc.z * inv) | ((uint32_t)f32_to_bf16_rne(acc.w * inv) << 16);
      *reinterpret_cast<uint2*>(p.out + ((size_t)(si.row0 + rr) * p.Hq + qh) * D + 4 * dq) = make_uint2(w0, w1);
    }
  }
}

template <int D, int G, int BS, bool F8>
hipError_t launch_decode_t(const AttnParams& p, hipStream_t stream) {
  const dim3 grid(p.decode_waves / p.decode_group), block(p.decode_group * kWave);
  const size_t lds = (size_t)p.decode_group * kTile * (D / 8) * 16;   // one bf16 tile per wave
  if (p.decode_max_q > 1)
    hipLaunchKernelGGL((decode_kernel<D, G, BS, true, F8>), grid, block, lds, stream, p);
  else
    hipLaunchKernelGGL((decode_kernel<D, G, BS, false, F8>), grid, block, lds, stream, p);
  return hipGetLastError();
}

// E4M3 rows of d 64 are 64 bytes: a wave-wide load covers 16 rows, more than an 8-slot block.
template <int D, bool F8>
constexpr bool decode_bs8_ok() { return !(F8 && D == 64); }

template <int D, int G, bool F8>
hipError_t dispatch_bs(const AttnParams& p, hipStream_t stream) {
  switch (p.bs) {
    case 8:
      if constexpr (decode_bs8_ok<D, F8>()) return launch_decode_t<D, G, 8, F8>(p, stream);
      break;
    case 16: return launch_decode_t<D, G, 16, F8>(p, stream);
    case 32: return launch_decode_t<D, G, 32, F8>(p, stream);
  }
  return hipErrorInvalidValue;
}

template <int D, bool F8>
hipError_t dispatch_g(const AttnParams& p, hipStream_t stream) {
  switch (p.Hq / p.Hkv) {
    case 1: return dispatch_bs<D, 1, F8>(p, stream);
    case 2: return dispatch_bs<D, 2, F8>(p, stream);
    case 4: return dispatch_bs<D, 4, F8>(p, stream);
    case 8: return dispatch_bs<D, 8, F8>(p, stream);
    case 16: return dispatch_bs<D, 16, F8>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_supported(int D, int G, int bs, bool fp8) {
  return (D == 64 || D == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16) &&
         (bs == 8 || bs == 16 || bs == 32) && !(fp8 && D == 64 && bs == 8);
}

hipError_t launch_decode(const AttnParams& p, bool fp8, hipStream_t stream) {
  if (fp8) {
    if (p.D == 128) return dispatch_g<128, true>(p, stream);
    if (p.D == 64) return dispatch_g<64, true>(p, stream);
  } else {
    if (p.D == 128) return dispatch_g<128, false>(p, stream);
    if (p.D == 64) return dispatch_g<64, false>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const AttnParams& p, hipStream_t stream) {
  // many pieces per (sequence, head) are possible only for long sequences: share a cell
  // among the waves of a workgroup there
  const int64_t cells = (int64_t)p.num_seqs * p.Hq;
  const bool wide = p.max_splits > 32;
  AttnParams q = p;
  q.merge_blocks = (int)(wide ? cells : (cells + kMergeWaves - 1) / kMergeWaves);
  // fused append: one more workgroup per 256 chunks of new rows (at most 4096; they stride)
  int64_t append_blocks = 0;
  if (p.k_new) {
    const int64_t chunks = p.num_q_tokens * 2 * ((int64_t)p.Hkv * p.D / 8);
    append_blocks = std::min<int64_t>((chunks + kMergeWaves * kWave - 1) / (kMergeWaves * kWave), 4096);
  }
  // the prefill planner rides along as the first workgroup when prefill rows are possible
  q.plan_first = p.max_query_len > p.decode_max_q ? 1 : 0;
  q.plan_bin_shift = 0;
  while ((((int64_t)p.max_blocks * p.bs + 63) / 64 >> q.plan_bin_shift) >= kPlanBins) ++q.plan_bin_shift;
  const dim3 grid((unsigned)(q.plan_first + q.merge_blocks + append_blocks));
  const dim3 block(kMergeWaves * kWave);
  if (p.D == 128) {
    if (wide) hipLaunchKernelGGL((merge_kernel<128, true>), grid, block, 0, stream, q);
    else hipLaunchKernelGGL((merge_kernel<128, false>), grid, block, 0, stream, q);
  } else if (p.D == 64) {
    if (wide) hipLaunchKernelGGL((merge_kernel<64, true>), grid, block, 0, stream, q);
    else hipLaunchKernelGGL((merge_kernel<64, false>), grid, block, 0, stream, q);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
