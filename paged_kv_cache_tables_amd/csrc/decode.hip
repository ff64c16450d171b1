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
//   * Partition (found by every wave from the lengths, with a wave scan; no
//     host work): the decode rows' work is cut into units (segment, group of
//     KV heads, 64-token tile), in that order.  A segment is a sequence's own tiles, or the tiles a group of
//     sequences maps to the same physical blocks (a shared prefix) for a block
//     of 16 query columns of its members.  The grid has one wave per resident
//     wave slot of the device; a workgroup holds one wave per KV head of a
//     group (up to 8) and takes an equal consecutive share of units, walked as
//     pieces of consecutive segments.  The waves of a workgroup read the same
//     slots for different heads, and a slot's heads sit side by side in the
//     pool, so the DRAM rows behind each slot are read together.
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
//   * Shared prefixes: a group piece takes its 16 columns from 16 / G member
//     sequences (one decode row each) and reads the shared tiles through the
//     leader's table.
//   A piece that covers a whole private segment of a sequence in no group
//   writes bf16 output directly; every other piece writes fp32 partials
//   (O, m, l) to the workspace, which the merge kernel combines.
#include <algorithm>
#include <climits>

#include "common.h"
#include "kernels.h"
#include "planner.h"
#include "rows.h"

namespace pkv {

namespace {

typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4v lds_short4;

// ---------------------------------------------------------------------------------------
// Shared prefixes.  Sequences of a batch can map the same physical blocks for a common
// prefix ("Under the Hood: PagedAttention", prefix sharing: one cached copy, several block
// tables pointing at it -- Text Generation Inference page; the radix prefix cache of the
// text-generation-inference v3 walkthrough builds such tables).  Attending that prefix once
// per sequence re-reads the same K/V.  Every decode workgroup first checks whether two decode
// sequences (one query row each) start with the same block: up to 64 sequences, each wave
// sorts the lanes' first blocks; beyond that, its waves fill one hash table in LDS together.
// If none do, the partition below is the plain per-sequence one.  If some do, every workgroup
// builds the same sharing plan in LDS (the tile buffers as scratch, a small region after
// them for the result): the sequences with a common first block form a group under the
// first of them (the leader); each member's block table is compared with the leader's,
// entry by entry, up to the cached full 64-token tiles of both; the group's shared run is
// the shortest such run among the members that share at least one tile.  Those tiles are
// then attended once per block of 16 query columns (16 / G members): group segments, read
// through the leader's table, placed after the sequences' own (private) segments, which
// skip them.  The merge kernel combines a member's private and group pieces.
// ---------------------------------------------------------------------------------------

// The plan's result, kept in LDS after the tile buffers for the whole kernel, for S
// sequences (Sr = S rounded up to a multiple of 4): [hdr 4][tiles skipped by each sequence
// Sr][members Sr][groups (leader, shared tiles, first member, members) Sr / 2 int4][group
// segment unit offsets Sr + 4][group segment (group, block) Sr int2] = 7 Sr + 8 ints.
struct SharePlan {
  int* hdr;         // [0] groups, [1] group segments, [2] units of all group segments
  int* tofs;        // per sequence: leading tiles attended by its group (0: not a member)
  int* members;     // member sequences, grouped, in sequence order within a group
  int4* grp;        // per group: (leader, shared tiles, first member slot, members)
  int* cboff;       // per group segment: first unit, relative to the first group unit
  int2* cbrec;      // per group segment: (group, column block within the group)
  __device__ SharePlan(int* base, int S) {
    const int Sr = (S + 3) & ~3;
    hdr = base;
    tofs = hdr + 4;
    members = tofs + Sr;
    grp = reinterpret_cast<int4*>(members + Sr);  // 16-byte aligned: 4 + 2 Sr ints, Sr % 4 == 0
    cboff = reinterpret_cast<int*>(grp + Sr / 2);
    cbrec = reinterpret_cast<int2*>(cboff + Sr + 4);
  }
};

// Exclusive prefix sum of one int per thread over the workgroup; `total` gets the sum.
__device__ int block_excl_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const int x = wave_tot[i];
    before += i < w ? x : 0;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return before + incl - v;
}

// Builds the sharing plan with every thread of the workgroup (each workgroup builds the same
// plan).  scratch: the tile buffers, at least 9 S + 2 hash_slots + 16 ints.
// NG = KV-head groups (units per tile).  Workgroup 0 also writes each sequence's group record
// for the merge kernel.
__device__ void build_share_plan(const AttnParams& p, int* scratch, const SharePlan& P, int NG, int G) {
  const int S = p.num_seqs, t = threadIdx.x, T = blockDim.x;
  const int HS = p.share_hash_slots;              // a power of two >= 2 S
  const int nblocks = p.num_blocks > INT_MAX ? INT_MAX : (int)p.num_blocks;
  const int bpt = kTile / p.bs;                   // pool blocks per tile
  int* hkey = scratch;                            // first block ids, -1 = empty
  int* hval = hkey + HS;                          // smallest sequence with that first block
  int* leader = hval + HS;                        // leader of a candidate, else -1
  int* tiles = leader + S;                        // hash slot, then tiles shared with the leader
  int* cnt = tiles + S;                           // per leader: candidates, then first group segment
  int* dtiles = cnt + S;                          // decode tiles of each sequence
  int* nmem = dtiles + S;                         // per leader: members
  int* gt = nmem + S;                             // per leader: shared tiles of the group
  int* mis = gt + S;                              // first block that differs from the leader's
  int* membase = mis + S;                         // per leader: first member slot
  int* cmp_list = membase + S;                    // [S] candidates whose tables are compared
  int* wave_tot = cmp_list + S;                   // [T / 64]

  // A: candidates (one decode row, at least one cached full tile -- its decode tiles minus
  // the tile of its newest token) keyed by their first block
  for (int i = t; i < HS; i += T) { hkey[i] = -1; hval[i] = INT_MAX; }
  for (int s = t; s < S; s += T) { leader[s] = -1; cnt[s] = 0; nmem[s] = 0; gt[s] = INT_MAX; mis[s] = INT_MAX; }
  __syncthreads();
  for (int s = t; s < S; s += T) {
    const int b0 = p.block_tables[(size_t)s * p.max_blocks];
    const SeqInfo si = seq_info(p, s);
    dtiles[s] = si.tiles;
    if (si.q != 1 || si.tiles < 2 || (unsigned)b0 >= (unsigned)nblocks) continue;
    unsigned h = ((unsigned)b0 * 2654435761u) & (unsigned)(HS - 1);
    for (int probe = 0; probe < HS; ++probe) {    // at most S keys in HS >= 2 S slots
      const int prev = atomicCAS(&hkey[h], -1, b0);
      if (prev == -1 || prev == b0) break;
      h = (h + 1) & (unsigned)(HS - 1);
    }
    atomicMin(&hval[h], s);
    tiles[s] = (int)h;
    leader[s] = -2;
  }
  __syncthreads();
  for (int s = t; s < S; s += T) {
    if (leader[s] != -2) continue;
    const int l = hval[tiles[s]];
    leader[s] = l;
    atomicAdd(&cnt[l], 1);
  }
  __syncthreads();
  // B: tiles each candidate shares with its leader
  for (int s = t; s < S; s += T) {
    const int l = leader[s];
    tiles[s] = (l >= 0 && cnt[l] >= 2) ? min(dtiles[s], dtiles[l]) - 1 : 0;
  }
  __syncthreads();
  // the candidates to compare (not leaders, at least one tile in common by length), listed in
  // cmp_list; then each wave takes batches of kCmpBatch of them, lane j comparing table entry
  // j0 + j of each (blocks 1 .. tiles * bpt - 1; block 0 is equal by construction), all of a
  // round's loads issued before any is checked
  int ncmp = 0;
  for (int c0 = 0; c0 < S; c0 += T) {
    const int s = c0 + t;
    const bool want = s < S && leader[s] >= 0 && leader[s] != s && tiles[s] > 0;
    int tot;
    const int idx = ncmp + block_excl_scan(want ? 1 : 0, wave_tot, tot);
    if (want) cmp_list[idx] = s;
    ncmp += tot;
  }
  __syncthreads();
  {
    constexpr int kCmpBatch = 16;
    const int lane = t & (kWave - 1), wv = t / kWave, nw = T / kWave;
    for (int base = wv * kCmpBatch; base < ncmp; base += nw * kCmpBatch) {
      int sm[kCmpBatch], lm[kCmpBatch], nbm[kCmpBatch];
      unsigned done = 0;
#pragma unroll
      for (int k = 0; k < kCmpBatch; ++k) {
        const int i = base + k;
        sm[k] = i < ncmp ? cmp_list[i] : 0;
        lm[k] = i < ncmp ? leader[sm[k]] : 0;
        nbm[k] = i < ncmp ? tiles[sm[k]] * bpt : 0;
        if (nbm[k] <= 1) done |= 1u << k;
      }
      for (int j0 = 1; done != (1u << kCmpBatch) - 1; j0 += kWave) {
        int va[kCmpBatch], vb[kCmpBatch];
#pragma unroll
        for (int k = 0; k < kCmpBatch; ++k) {
          const int j = j0 + lane;
          const bool act = !(done >> k & 1) && j < nbm[k];
          va[k] = act ? p.block_tables[(size_t)sm[k] * p.max_blocks + j] : 0;
          vb[k] = act ? p.block_tables[(size_t)lm[k] * p.max_blocks + j] : 0;
        }
#pragma unroll
        for (int k = 0; k < kCmpBatch; ++k) {
          if (done >> k & 1) continue;
          const unsigned long long d = __builtin_amdgcn_ballot_w64(j0 + lane < nbm[k] && va[k] != vb[k]);
          if (d) {
            if (lane == 0) mis[sm[k]] = j0 + (int)__builtin_ctzll(d);
            done |= 1u << k;
          } else if (j0 + kWave >= nbm[k]) {
            done |= 1u << k;
          }
        }
      }
    }
  }
  __syncthreads();
  for (int s = t; s < S; s += T)
    if (leader[s] >= 0 && leader[s] != s && mis[s] != INT_MAX) tiles[s] = min(tiles[s], mis[s] / bpt);
  __syncthreads();
  // C: a group = its candidates sharing at least one tile (the leader among them); its shared
  // run is the shortest of theirs
  for (int s = t; s < S; s += T) {
    const int l = leader[s];
    if (l >= 0 && tiles[s] >= 1) {
      atomicMin(&gt[l], tiles[s]);
      atomicAdd(&nmem[l], 1);
    }
  }
  __syncthreads();
  auto is_member = [&](int s) {
    const int l = leader[s];
    return l >= 0 && tiles[s] >= 1 && nmem[l] >= 2;
  };
  // D: groups in leader order; each group's column blocks are its segments
  int ngroups = 0, ncb = 0, nmembers = 0;
  for (int c0 = 0; c0 < S; c0 += T) {
    const int s = c0 + t;
    const bool lead = s < S && leader[s] == s && nmem[s] >= 2;
    const int ng = lead ? nmem[s] : 0;
    const int nc = (ng * G + 15) / 16;
    int tg, tc, tm;
    const int gi = ngroups + block_excl_scan(lead ? 1 : 0, wave_tot, tg);
    const int cbb = ncb + block_excl_scan(nc, wave_tot, tc);
    const int mb = nmembers + block_excl_scan(ng, wave_tot, tm);
    if (lead) {
      cnt[s] = cbb;
      membase[s] = mb;
      P.grp[gi] = make_int4(s, gt[s], mb, ng);
      for (int cb = 0; cb < nc; ++cb) P.cbrec[cbb + cb] = make_int2(gi, cb);
    }
    ngroups += tg;
    ncb += tc;
    nmembers += tm;
  }
  __syncthreads();
  // members in sequence order within each group: wave 0 walks the sequences 64 at a time,
  // ranking the members of each group present with a ballot and a running count per leader
  // (in mis, free by now); a member's columns are (rank G .. + G - 1) of its group, in column
  // block (rank G) / 16
  for (int s = t; s < S; s += T) mis[s] = 0;     // running member count per leader
  __syncthreads();
  if (t < kWave) {
    for (int c0 = 0; c0 < S; c0 += kWave) {
      const int s = c0 + t;
      const int l = (s < S && is_member(s)) ? leader[s] : -1;
      unsigned long long left = __builtin_amdgcn_ballot_w64(l >= 0);
      while (left) {
        const int src = (int)__builtin_ctzll(left);
        const int lg = __shfl(l, src, kWave);
        const unsigned long long m = __builtin_amdgcn_ballot_w64(l == lg);
        const int before = mis[lg];
        if (l == lg) {
          const int rank = before + (int)__builtin_popcountll(m & ((1ull << t) - 1));
          tiles[s] = -1 - rank;                  // the rank, marked (tiles is no longer needed)
        }
        wave_lds_sync();
        if (t == src) mis[lg] = before + (int)__builtin_popcountll(m);
        wave_lds_sync();
        left &= ~m;
      }
    }
  }
  __syncthreads();
  for (int s = t; s < S; s += T) {
    int2 rec = make_int2(-1, 0);
    int skip = 0;
    if (tiles[s] < 0) {                          // a member: tiles holds -1 - rank
      const int l = leader[s], rank = -1 - tiles[s];
      P.members[membase[l] + rank] = s;
      rec = make_int2(S + cnt[l] + rank * G / 16, (rank * G) % 16);
      skip = gt[l];
    }
    P.tofs[s] = skip;
    if (blockIdx.x == 0) p.plan_memrec[s] = rec;
  }
  __syncthreads();
  // group segment offsets (units: NG per shared tile)
  int run = 0;
  for (int c0 = 0; c0 < ncb; c0 += T) {
    const int k = c0 + t;
    const int u = k < ncb ? NG * P.grp[P.cbrec[k].x].y : 0;
    int tt;
    const int off = run + block_excl_scan(u, wave_tot, tt);
    if (k < ncb) P.cboff[k] = off;
    run += tt;
  }
  if (t == 0) {
    P.cboff[ncb] = run;
    P.hdr[0] = ngroups;
    P.hdr[1] = ncb;
    P.hdr[2] = run;
  }
  __syncthreads();
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

  // ---- the partition: units (segment, head group, tile) in that order, an equal share per
  // workgroup.  Segments: each sequence's own tiles (those its sharing group does not attend
  // for it), then the sharing groups' column blocks.  The waves of a workgroup take the same
  // units for the heads of one group, so the heads' rows of each pool slot (adjacent in memory)
  // are read at the same time.  Lane l sums the tiles of sequences [l c, (l + 1) c); a wave
  // scan gives each lane the units before its chunk.  Unit counts fit in 32 bits (checked by
  // the host). ----
  const int S = p.num_seqs;
  const int c_per = (S + kWave - 1) / kWave;
  // sharing check, by all waves of the workgroup together: the candidates' first blocks in one
  // hash table (share_hash_slots >= 2 S entries, a power of two) at the start of wave 0's tile
  // buffer, each wave inserting every WPG-th element of the lanes' chunks; a wave that finds a
  // repeated block sets an LDS flag
  // With at most 64 sequences (one per lane) each wave instead sorts the lanes' first blocks
  // and compares neighbours: no table, no barrier.
  const bool detect = p.share_seqs > 0;
  const bool wave_check = detect && c_per == 1;
  const bool table_check = detect && !wave_check;
  __shared__ int share_flag;
  int* whash = reinterpret_cast<int*>(lds_tiles);
  const int HS = p.share_hash_slots;
  int wkey = -1 - lane;                          // the lane's candidate key (a distinct negative one if none)
  if (table_check) {
    for (int i = threadIdx.x; i < HS / 4; i += (int)blockDim.x) reinterpret_cast<uint4*>(whash)[i] = make_uint4(~0u, ~0u, ~0u, ~0u);
    if (threadIdx.x == 0) share_flag = 0;
    __syncthreads();                             // the table is clear
  }
  const int nblocks_i = p.num_blocks > 0x7fffffff ? 0x7fffffff : (int)p.num_blocks;
  int my_tiles = 0;
  bool dup = false;
  SeqInfo first{0, 0, 0, 0};                     // this lane's first sequence
  // the lane's sequences in batches, every load of a batch issued before any is used
  constexpr int kSeqBatch = 8;
  for (int i0 = 0; i0 < c_per; i0 += kSeqBatch) {
    SeqInfo si[kSeqBatch];
    int b0[kSeqBatch];
#pragma unroll
    for (int k = 0; k < kSeqBatch; ++k) {
      const int s = lane * c_per + i0 + k;
      const bool ok = i0 + k < c_per && s < S;
      si[k] = ok ? seq_info(p, s) : SeqInfo{0, 0, 0, 0};
      b0[k] = (ok && (wave_check || (table_check && (i0 + k) % WPG == wv))) ? p.block_tables[(size_t)s * p.max_blocks] : -1;
    }
    if (i0 == 0) first = si[0];
#pragma unroll
    for (int k = 0; k < kSeqBatch; ++k) {
      my_tiles += si[k].tiles;
      const bool cand = si[k].q == 1 && si[k].tiles >= 2 && (unsigned)b0[k] < (unsigned)nblocks_i;
      if (wave_check && k == 0 && cand) wkey = b0[k];
      if (table_check && cand) {                 // (b0 only for this wave's elements)
        unsigned h = ((unsigned)b0[k] * 2654435761u) & (unsigned)(HS - 1);
        for (int probe = 0; probe < HS; ++probe) {   // at most S keys in HS >= 2 S slots
          const int prev = atomicCAS(&whash[h], -1, b0[k]);
          if (prev == -1) break;
          if (prev == b0[k]) { dup = true; break; }
          h = (h + 1) & (unsigned)(HS - 1);
        }
      }
    }
  }
  bool sharing = false;
  if (wave_check) {
    // bitonic sort of the 64 keys across the lanes (ascending), then equal neighbours
#pragma unroll
    for (int kk = 2; kk <= kWave; kk <<= 1)
#pragma unroll
      for (int j = kk >> 1; j > 0; j >>= 1) {
        const int o = __shfl_xor(wkey, j, kWave);
        const bool keep_min = ((lane & j) == 0) == ((lane & kk) == 0);
        wkey = keep_min ? min(wkey, o) : max(wkey, o);
      }
    const int prev = __shfl_up(wkey, 1, kWave);
    sharing = __builtin_amdgcn_ballot_w64(lane > 0 && wkey >= 0 && prev == wkey) != 0;
  } else if (table_check) {
    const bool any_dup = __builtin_amdgcn_ballot_w64(dup) != 0;
    if (any_dup && lane == 0) share_flag = 1;
    __syncthreads();                             // every insert and flag write is done
    sharing = uniform(share_flag) != 0;
  }
  if (detect && !sharing && w == 0)              // no group: the merge kernel sees no member
    for (int i = threadIdx.x; i < S; i += blockDim.x) p.plan_memrec[i] = make_int2(-1, 0);
  const SharePlan P(reinterpret_cast<int*>(lds_tiles + (size_t)WPG * kTile * CH), S);
  if (sharing) {
    build_share_plan(p, reinterpret_cast<int*>(lds_tiles), P, NG, G);
    for (int i = 0; i < c_per; ++i) {
      const int s = lane * c_per + i;
      if (s < S) my_tiles -= P.tofs[s];
    }
  }
  const int incl = wave_incl_scan(my_tiles);
  const int priv_units_total = uniform(__shfl(incl, kWave - 1, kWave) * NG);   // NG x private tiles
  const int total_units = priv_units_total + (sharing ? uniform(P.hdr[2]) : 0);
  if (total_units == 0) return;
  const int nwg = p.decode_waves / WPG;          // workgroups of the grid
  const int share = uniform(max(p.min_share_tiles, (total_units + nwg - 1) / nwg));
  if (w >= (total_units + share - 1) / share) return;   // fewer shares than workgroups
  const int x0 = w * share;
  const int x1 = min(x0 + share, total_units);

  // The current segment.  Private: sequence s, its rows (cur_row0, cur_q) and length, tiles
  // [t_off, t_off + nt).  Group column block k (segment S + k): s = the group's leader (whose
  // table is read), cur_q = -1 - k, cur_len = the shared keys, nt = the shared tiles, t_off = 0;
  // the block's members come from the plan in LDS when a piece needs them.
  int s = 0, seg_a = 0, cur_row0 = 0, cur_q = 0, cur_len = 0, nt = 0, t_off = 0;
  auto load_cb = [&](int k) {
    const int4 gr = P.grp[P.cbrec[k].x];
    s = uniform(gr.x);
    nt = uniform(gr.y);
    cur_len = nt * kTile;
    cur_q = -1 - k;
    cur_row0 = 0;
    t_off = 0;
  };
  if (x0 < priv_units_total) {
    // the lane whose chunk holds unit x0, then the sequence inside that chunk
    const int excl_units = (incl - my_tiles) * NG;
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(excl_units <= x0 && x0 < incl * NG);
    const int src = (int)__builtin_ctzll(hit);   // nonempty: x0 < priv_units_total
    s = uniform(src * c_per);
    seg_a = uniform(__shfl(excl_units, src, kWave));   // first unit of sequence s
    cur_row0 = uniform(__shfl(first.row0, src, kWave));
    cur_q = uniform(__shfl(first.q, src, kWave));
    cur_len = uniform(__shfl(first.len, src, kWave));
    t_off = sharing ? uniform(P.tofs[s]) : 0;
    nt = uniform(__shfl(first.tiles, src, kWave)) - t_off;
  } else {
    // a group segment: the last one whose first unit is <= x0
    const int y = x0 - priv_units_total;
    int lo = 0, hi = uniform(P.hdr[1]) - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (uniform(P.cboff[mid]) <= y) lo = mid; else hi = mid - 1;
    }
    seg_a = priv_units_total + uniform(P.cboff[lo]);
    load_cb(lo);
  }
  auto next_seg = [&]() {
    seg_a += NG * nt;
    if (cur_q < 0) {                             // the next group segment
      load_cb(-cur_q);
    } else if (s + 1 < S) {                      // the next sequence
      s = uniform(s + 1);
      const SeqInfo si = seq_info(p, s);
      cur_row0 = uniform(si.row0);
      cur_q = uniform(si.q);
      cur_len = uniform(si.len);
      t_off = sharing ? uniform(P.tofs[s]) : 0;
      nt = uniform(si.tiles) - t_off;
    } else {                                     // past the last sequence: the group segments
      load_cb(0);
    }
  };
  while (cur_q >= 0 && x0 >= seg_a + NG * nt && s + 1 < S) next_seg();

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

  // One piece: tiles [tb0, tb1) of the current segment for KV head h, whose units start at
  // unit a.
  auto piece = [&](int h, int tb0, int tb1, int a) {
    const bool grp = cur_q < 0;                  // a group segment's piece
    const int row0 = cur_row0;
    const int L = cur_len;
    const int g = n % G;
    // accumulator column n: in a private piece (row rr of the sequence's q_s rows, head g),
    // the row at position L - q_s + rr attends keys 0..lim; in a group piece (member
    // cb 16 / G + n / G, head g), whose decode row sees every shared key
    int qrow = 0, lim = INT_MAX;
    bool col_valid;
    if (grp) {
      const int2 cr = P.cbrec[-1 - cur_q];       // (group, column block)
      const int4 gr = P.grp[cr.x];               // (leader, shared tiles, first member, members)
      const int mi = cr.y * (16 / G) + n / G;
      col_valid = mi < gr.w;
      if (col_valid) qrow = p.qsl[P.members[gr.z + mi]];
    } else {
      const int rr = n / G;
      col_valid = rr < cur_q;
      qrow = row0 + (col_valid ? rr : 0);
      lim = col_valid ? L - cur_q + rr : L - 1;
    }
    const int t_begin = uniform((t_off + tb0) * kTile);
    const int t_end = uniform(min((t_off + tb1) * kTile, L));
    const int* bt_row = p.block_tables + (size_t)s * p.max_blocks;
    const char* kbase = p.k_cache + (size_t)h * D * EB;
    const char* vbase = p.v_cache + (size_t)h * D * EB;
    // positions fresh0 .. L - 1 are this step's tokens; with a fused append they are not in
    // the pools yet and come from the rows of k_new / v_new instead (never in shared tiles)
    const int fresh0 = uniform((!F8 && !grp && p.k_new != nullptr) ? L - cur_q : INT_MAX);
    const uint16_t* knew_h = p.k_new + (size_t)h * D;
    const uint16_t* vnew_h = p.v_new + (size_t)h * D;

    // ---- Q^T as the B operand: column n, dims ks*32 + kg*8 .. +8 (zero for padding columns) ----
    bf16x8 qreg[KS];
    {
      const uint16_t* qp = p.q + ((size_t)qrow * Hq + (size_t)h * G + g) * D;
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

    // Block-table entries of a tile (wave-uniform loads).  Entries past the end, or outside
    // the pool, become block 0: a safe address whose rows the masks ignore.  For 8-bit pools
    // they come through the scalar cache, so the wait for them is not a wait for the tile
    // loads in flight (measured: Llama-3-8B batch 74 -> 68 us per call; for bf16 pools the
    // vector form measured 2-3% faster on the 70B and long-context batches).
    auto load_bts = [&](int t0, int* dst) {
#pragma unroll
      for (int j = 0; j < NBT; ++j) {
        const int e = uniform((t0 + j * BS) / BS);
        const int b = (t0 + j * BS < t_end) ? (F8 ? load_uniform_int(bt_row, e) : bt_row[e]) : 0;
        dst[j] = (unsigned)b < (unsigned)nblocks ? b : 0;
      }
    };
    // Coalesced tile load: load i covers rows RPI*i .. RPI*i + RPI - 1 (one pool block), with the
    // streaming hint.  A tile that holds fresh positions takes those rows from the new rows
    // instead (lane by lane).
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
    const int g_e = n_e % G;
    const int qh = h * G + g_e;
    const int first_w = a / share;                 // the workgroup holding tile 0 of (segment, h)
    const int nseg = (a + nt - 1) / share - first_w + 1;   // pieces of (segment, h)
    // partial slot: 2 w for the piece that opens this workgroup's share, 2 w + 1 for a later one
    // (only the last piece of a share can be a later partial one)
    const int slot = 2 * w + (a + tb0 != x0 ? 1 : 0);
    const int seg_k = grp ? S - 1 - cur_q : s;   // the segment's record: sequence s, or S + block
    if (tb0 == 0 && lane == 0) p.ws_nparts[(size_t)seg_k * Hkv + h] = make_int2(slot, nseg);
    float l_tot = l_part + __shfl_xor(l_part, 16, kWave);
    l_tot += __shfl_xor(l_tot, 32, kWave);
    // where column n_e goes: final output (a whole private segment of a sequence in no group),
    // the sequence's own row for a whole segment of a group member, or a slot row
    int64_t prow = -1;                            // partial row, or -1
    int out_row = -1;                             // query row of a final output, or -1
    if (grp) {
      const int2 cr = P.cbrec[-1 - cur_q];
      const int4 gr = P.grp[cr.x];
      const int mi = cr.y * (16 / G) + n_e / G;
      if (mi < gr.w) {
        const int s_e = P.members[gr.z + mi];
        prow = nseg == 1 ? p.mem_rows0 + (int64_t)(p.share_seqs + s_e) * Hq + qh
                         : ((int64_t)slot * WPG + wv) * 16 + n_e;
      }
    } else {
      const int rr_e = n_e / G;
      if (rr_e < cur_q) {
        if (nseg > 1) prow = ((int64_t)slot * WPG + wv) * 16 + n_e;
        else if (t_off > 0) prow = p.mem_rows0 + (int64_t)s * Hq + qh;   // a group member's own tiles
        else out_row = row0 + rr_e;
      }
    }
    if (out_row >= 0) {                            // the whole (s, h): final output
      const float inv = F8 ? p.v_scale / l_tot : 1.f / l_tot;
      uint16_t* op = p.out + ((size_t)out_row * Hq + qh) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint32_t w0 = pack_bf16x2(oacc[db][0] * inv, oacc[db][1] * inv);
        const uint32_t w1 = pack_bf16x2(oacc[db][2] * inv, oacc[db][3] * inv);
        *reinterpret_cast<uint2*>(op + db * 16 + 4 * kg_e) = make_uint2(w0, w1);
      }
    } else if (prow >= 0) {                        // a partial for the merge kernel
      const float vs = F8 ? p.v_scale : 1.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<float4*>(p.ws_o + prow * D + db * 16 + 4 * kg_e) =
            make_float4(oacc[db][0] * vs, oacc[db][1] * vs, oacc[db][2] * vs, oacc[db][3] * vs);
      if (kg_e == 0) { p.ws_m[prow] = m_run; p.ws_l[prow] = l_tot; }
    }
  };

  // ---- walk the share: pieces of consecutive segments; this wave takes the head wv of each
  // head group ----
  int pos = x0;
  while (pos < x1) {
    if (pos >= seg_a + NG * nt) {                // past the current segment (or an empty one)
      next_seg();
      continue;
    }
    const int hg = (pos - seg_a) / nt;
    const int a = seg_a + hg * nt;               // first unit of (segment, hg)
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
  // the records of the sequence's own segment (segment s) and of its sharing group are loaded
  // together with the lengths; they are used only for sequences with decode rows, whose
  // records the decode kernel wrote
  const int2 prv = p.ws_nparts[(size_t)s * p.Hkv + h];
  const int2 mrec = p.share_seqs > 0 ? p.plan_memrec[s] : make_int2(-1, 0);
  const SeqInfo si = seq_info(p, s);
  if (si.tiles == 0) return;                     // no decode rows (or nothing to attend)
  const bool member = mrec.x >= 0;               // a member of a prefix-sharing group
  if (!member && prv.y <= 1) return;             // written directly by the decode kernel
  const int2 grp = member ? p.ws_nparts[(size_t)mrec.x * p.Hkv + h] : make_int2(0, 0);
  const int nA = prv.y, nB = member ? grp.y : 0;
  const int nsplit = nA + nB;
  // partial row of piece j of decode row rr: the pieces of the sequence's own segment (the
  // first in slot prv.x, piece j > 0 in slot 0 of the j-th following workgroup; a member's
  // whole segment in its own row), then those of its group's column block
  const int64_t slot_rows = (int64_t)p.decode_group * 16;
  const int64_t stride = 2 * slot_rows;          // from slot 0 of one workgroup to the next
  const int64_t colA = wv_h * 16 + g, colB = wv_h * 16 + mrec.y + g;
  const int64_t a0 = (member && nA == 1) ? p.mem_rows0 + (int64_t)s * p.Hq + qh : prv.x * slot_rows + colA;
  const int64_t a1 = (int64_t)(prv.x / 2 + 1) * stride + colA;
  const int64_t b0 = nB == 1 ? p.mem_rows0 + (int64_t)(p.share_seqs + s) * p.Hq + qh : grp.x * slot_rows + colB;
  const int64_t b1 = (int64_t)(grp.x / 2 + 1) * stride + colB;
  auto piece_row = [&](int j, int rr) -> int64_t {
    const int64_t r = j < nA ? (j == 0 ? a0 : a1 + (int64_t)(j - 1) * stride)
                             : (j == nA ? b0 : b1 + (int64_t)(j - nA - 1) * stride);
    return r + rr * G;                           // decode row rr: column rr G + g (sequences in no group)
  };
  if constexpr (!WIDE) {
    // One pass with a running max, CK wave-wide steps (PPI pieces each) of loads in flight
    // at a time; lanes past the piece count load nothing and are discarded by selection,
    // never by a zero weight.
    constexpr int CK = 4;
    auto merge_row = [&](int rr, int row0) {
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
            const int64_t r = piece_row(j, rr);
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
        const uint32_t w0 = pack_bf16x2(acc.x * inv, acc.y * inv);
        const uint32_t w1 = pack_bf16x2(acc.z * inv, acc.w * inv);
        *reinterpret_cast<uint2*>(p.out + ((size_t)(row0 + rr) * p.Hq + qh) * D + 4 * dq) = make_uint2(w0, w1);
      }
    };
    for (int rr = 0; rr < si.q; ++rr) merge_row(rr, si.row0);
    return;
  }
  const int w_in = WIDE ? wv : 0;

  for (int rr = 0; rr < si.q; ++rr) {
    float M = -INFINITY;                         // every wave of the cell finds the same M
    for (int j = lane; j < nsplit; j += kWave) M = fmaxf(M, p.ws_m[piece_row(j, rr)]);
    M = wave_max(M);

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float ls = 0.f;
#pragma unroll 4
    for (int j = w_in * PPI + sub; j < nsplit; j += WPC * PPI) {
      const int64_t r = piece_row(j, rr);
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
      const uint32_t w0 = pack_bf16x2(acc.x * inv, acc.y * inv);
      const uint32_t w1 = pack_bf16x2(acc.z * inv, acc.w * inv);
      *reinterpret_cast<uint2*>(p.out + ((size_t)(si.row0 + rr) * p.Hq + qh) * D + 4 * dq) = make_uint2(w0, w1);
    }
  }
}

template <int D, int G, int BS, bool F8>
hipError_t launch_decode_t(const AttnParams& p, hipStream_t stream) {
  const dim3 grid(p.decode_waves / p.decode_group), block(p.decode_group * kWave);
  // one bf16 tile per wave, then the sharing plan when the call is checked for shared prefixes
  const size_t lds = (size_t)p.decode_group * kTile * (D / 8) * 16 +
                     (p.share_seqs > 0 ? (size_t)share_plan_ints(p.share_seqs) * 4 : 0);
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
