// Prefill work list of one attention call, built by the first workgroup of the merge launch
// (which runs after the decode kernel and before the prefill kernel on the same stream).
#pragma once

#include "common.h"
#include "kernels.h"

namespace pkv {

// Buckets of the counting sort: entry tile counts are shifted right by plan_bin_shift so
// that the largest fits.
constexpr int kPlanBins = kPlanBinsHost;

// Sum of one int64 per thread over the workgroup (every thread gets it).
template <int THREADS>
__device__ int64_t plan_block_sum(int64_t v) {
  __shared__ int64_t part[THREADS / kWave];
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
#pragma unroll
  for (int d = 1; d < kWave; d *= 2) v += __shfl_xor(v, d, kWave);
  __syncthreads();                               // earlier readers of part are done
  if (lane == 0) part[w] = v;
  __syncthreads();
  int64_t tot = 0;
  for (int i = 0; i < THREADS / kWave; ++i) tot += part[i];
  return tot;
}

// Pieces of an item of `tiles` key tiles for split length T (1: not split), and their length
// (T < tiles < 2^25 when split: 32-bit division, the 64-bit one being a long software routine).
__device__ __forceinline__ int plan_pieces(int tiles, int T) {
  if (tiles <= T) return 1;
  const uint32_t n = ((uint32_t)tiles + (uint32_t)T - 1) / (uint32_t)T;
  return n < (uint32_t)kMaxPieces ? (int)n : kMaxPieces;
}
__device__ __forceinline__ int plan_piece_tiles(int tiles, int n) {
  return n == 1 ? tiles : (int)(((uint32_t)tiles + n - 1) / (uint32_t)n);
}

// Lists the prefill work of one call (the same list serves every KV head), longest first.  A
// sequence with q_s > decode_max_q rows (fewer are computed as decode rows) has
// ceil(q_s / rows_per_tile) row tiles; row tile mt needs the keys before position
// L - q_s + min((mt + 1) rows_per_tile, q_s), i.e. that many keys / 64 tiles of work.
//
// When the items are too few for the device (fewer per KV head than the prefill workgroups
// resident per head, e.g. a chunk over a long prefix), long items are cut along the keys, as
// decode rows are: an item of t > T tiles becomes n = ceil(t / T) pieces
// (at most kMaxPieces) of consecutive tiles, each attended by its own workgroup, which writes
// (O, m, l) partials; the last piece to finish merges them.  T = max(kSplitMinTiles,
// ceil(tiles of all items / slots per head)), doubled when the pieces would need more
// partial slots than the workspace holds (with the doubled T they never do: a split item has
// more than T tiles, so the pieces of split items number at most 2 tiles / T).
//
// Workgroups start in id order as earlier ones finish, so listing the entries by decreasing
// work is the longest-processing-time-first schedule: the long items (late row tiles of long
// prefixes) are not left to start last.  A counting sort over the entries' tile counts;
// entries of one bucket in any order.  The sequences with chunk rows are first gathered into
// a list in LDS (up to kPlanListCap of them) with the index of each one's first item, so
// that every later pass hands the items out one per thread; a batch with more of them walks
// its sequences one per thread.
// bins: kPlanBins ints of LDS; wave_tot: THREADS / 64 ints of LDS.
constexpr int kPlanListCap = 256;

template <int THREADS>
__device__ void plan_prefill_items(const AttnParams& p, int* bins, int* wave_tot) {
  static_assert(kPlanBins % THREADS == 0, "each thread owns whole bins");
  static_assert(THREADS == kPlanListCap, "one thread per listed sequence in the scan");
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  const int rows_per_tile = kPrefillPairs / (p.Hq / p.Hkv);
  const int max_len = p.max_blocks * p.bs;
  const int min_rows = p.decode_max_q;
  const int bin_shift = p.plan_bin_shift;
  __shared__ int4 seq_list[kPlanListCap];        // (sequence, prior keys, rows, row tiles)
  __shared__ int n_list;                         // sequences with chunk rows
  __shared__ int any_long;                       // some item has more than kSplitMinTiles tiles
  __shared__ int slot_next;                      // partial slots handed out so far (per head)
  for (int i = t; i < kPlanBins; i += THREADS) bins[i] = 0;
  if (t == 0) { n_list = 0; any_long = 0; slot_next = 0; }
  __syncthreads();
  auto item_tiles = [&](int prior, int q, int mt) -> int {   // key tiles of row tile mt
    const int key_end = prior + min((mt + 1) * rows_per_tile, q);
    return (max(key_end, 1) + 63) / 64;
  };
  // pass 0: the sequences with chunk rows (their last row tile is their longest item)
  for (int s = t; s < p.num_seqs; s += THREADS) {
    const int q = p.qsl[s + 1] - p.qsl[s];
    const int prior = min(p.seq_lens[s], max_len) - q;
    const int nt = q > min_rows ? (q + rows_per_tile - 1) / rows_per_tile : 0;
    if (nt > 0) {
      const int i = atomicAdd(&n_list, 1);
      if (i < kPlanListCap) seq_list[i] = make_int4(s, prior, q, nt);
      if (item_tiles(prior, q, nt - 1) > kSplitMinTiles) any_long = 1;
    }
  }
  __syncthreads();
  const int n_seq = n_list;
  // the listed sequences' first items: an exclusive scan of their row tiles
  __shared__ int item_base[kPlanListCap];
  int n_items = 0;
  if (n_seq <= kPlanListCap) {
    const int nt = t < n_seq ? seq_list[t].w : 0;
    int incl = nt;
#pragma unroll
    for (int d = 1; d < kWave; d *= 2) {
      const int y = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += y;
    }
    if (lane == kWave - 1) wave_tot[w] = incl;
    __syncthreads();
    int base = incl - nt;
    for (int i = 0; i < w; ++i) base += wave_tot[i];
    for (int i = 0; i < THREADS / kWave; ++i) n_items += wave_tot[i];
    if (t < n_seq) item_base[t] = base;
    __syncthreads();                             // item_base is written; wave_tot may be reused
  }
  // f(s, prior, q, mt) for every item (sequence s, row tile mt), spread over the threads
  auto for_items = [&](auto&& f) {
    if (n_seq <= kPlanListCap) {
      for (int i = t; i < n_items; i += THREADS) {
        int lo = 0, hi = n_seq - 1;              // the last sequence whose first item is <= i
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (item_base[mid] <= i) lo = mid; else hi = mid - 1;
        }
        const int4 sq = seq_list[lo];
        f(sq.x, sq.y, sq.z, i - item_base[lo]);
      }
    } else {
      for (int s = t; s < p.num_seqs; s += THREADS) {
        const int q = p.qsl[s + 1] - p.qsl[s];
        const int prior = min(p.seq_lens[s], max_len) - q;
        const int nt = q > min_rows ? (q + rows_per_tile - 1) / rows_per_tile : 0;
        for (int mt = 0; mt < nt; ++mt) f(s, prior, q, mt);
      }
    }
  };
  // bucket of an entry of `tiles` tiles: longest first
  auto bucket = [&](int tiles) { return kPlanBins - 1 - min(tiles >> bin_shift, kPlanBins - 1); };
  // the split length T (INT_MAX: nothing is split)
  int T = INT_MAX;
  if (any_long) {
    int64_t my_tiles = 0, my_items = 0;
    for_items([&](int, int prior, int q, int mt) {
      my_tiles += item_tiles(prior, q, mt);
      ++my_items;
    });
    const int64_t total = plan_block_sum<THREADS>(my_tiles);
    const int slots_h = max(1, min(p.prefill_slots, p.prefill_piece_cap) / p.Hkv);
    // with items enough to occupy every slot the longest-first order balances them, and
    // splitting would only add partials
    if (plan_block_sum<THREADS>(my_items) < slots_h) {
      const int cap_h = p.prefill_piece_cap / p.Hkv;   // partial slots of one head
      const int64_t T64 = (total + slots_h - 1) / slots_h;
      T = T64 < kSplitMinTiles ? kSplitMinTiles : (T64 > INT_MAX / 2 ? INT_MAX / 2 : (int)T64);
      int64_t my_split = 0;
      const int T1 = T;
      for_items([&](int, int prior, int q, int mt) {
        const int n = plan_pieces(item_tiles(prior, q, mt), T1);
        if (n > 1) my_split += n;
      });
      if (plan_block_sum<THREADS>(my_split) > cap_h) T *= 2;
    }
  }
  // pass 1: the entries' buckets (an item of n pieces: n entries of its piece length)
  const int Tc = T;
  for_items([&](int, int prior, int q, int mt) {
    const int tiles = item_tiles(prior, q, mt), n = plan_pieces(tiles, Tc);
    atomicAdd(&bins[bucket(plan_piece_tiles(tiles, n))], n);
  });
  __syncthreads();
  // exclusive scan of the bins: thread t owns bins [PER t, PER t + PER)
  constexpr int PER = kPlanBins / THREADS;
  int sum = 0;
  for (int i = 0; i < PER; ++i) sum += bins[PER * t + i];
  int incl = sum;
#pragma unroll
  for (int d = 1; d < kWave; d *= 2) {
    const int y = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += y;
  }
  if (lane == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  int run = incl - sum;
  for (int i = 0; i < w; ++i) run += wave_tot[i];
  int total_entries = 0;
  for (int i = 0; i < THREADS / kWave; ++i) total_entries += wave_tot[i];
  for (int i = 0; i < PER; ++i) {
    const int c = bins[PER * t + i];
    bins[PER * t + i] = run;
    run += c;
  }
  __syncthreads();
  // pass 2: the entries; a split item takes n partial slots and clears its counters
  for_items([&](int s, int prior, int q, int mt) {
    const int tiles = item_tiles(prior, q, mt), n = plan_pieces(tiles, Tc);
    const int pos = atomicAdd(&bins[bucket(plan_piece_tiles(tiles, n))], n);   // its pieces side by side
    int slot0 = 0;
    if (n > 1) {
      slot0 = atomicAdd(&slot_next, n);          // below the slots of one head by the choice of T
      for (int h = 0; h < p.Hkv; ++h) p.plan_split_ctr[(size_t)slot0 * p.Hkv + h] = 0;
    }
    for (int j = 0; j < n; ++j)
      if (pos + j < p.plan_capacity) p.plan_items[pos + j] = make_int4(s, mt, j | (n << 16), slot0);
  });
  if (t == 0) *p.plan_count = min(total_entries, p.plan_capacity);
}

}  // namespace pkv
