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

// The split length of a call with items longer than kSplitMinTiles, and the buckets rebuilt
// by piece length (n entries per item).
template <int THREADS>
__device__ __forceinline__ int plan_split_length(const AttnParams& p, int* bins) {
  const int t = threadIdx.x;
  const int rows_per_tile = kPrefillPairs / (p.Hq / p.Hkv);
  const int max_len = p.max_blocks * p.bs;
  const int min_rows = p.decode_max_q;
  const int bin_shift = p.plan_bin_shift;
  auto seq_tiles = [&](int s, int& prior, int& q) -> int {
    q = p.qsl[s + 1] - p.qsl[s];
    prior = min(p.seq_lens[s], max_len) - q;
    return q > min_rows ? (q + rows_per_tile - 1) / rows_per_tile : 0;
  };
  auto item_tiles = [&](int prior, int q, int mt) -> int {
    const int key_end = prior + min((mt + 1) * rows_per_tile, q);
    return (max(key_end, 1) + 63) / 64;
  };
  auto bucket = [&](int tiles) { return kPlanBins - 1 - min(tiles >> bin_shift, kPlanBins - 1); };
  int64_t my_tiles = 0, my_items = 0;
  for (int s = t; s < p.num_seqs; s += THREADS) {
    int prior, q;
    const int nt = seq_tiles(s, prior, q);
    my_items += nt;
    for (int mt = 0; mt < nt; ++mt) my_tiles += item_tiles(prior, q, mt);
  }
  const int64_t total = plan_block_sum<THREADS>(my_tiles);
  const int slots_h = max(1, min(p.prefill_slots, p.prefill_piece_cap) / p.Hkv);
  // items enough to occupy every slot: the longest-first order balances them, splitting would
  // only add partials (uniform: every thread has the sum)
  if (plan_block_sum<THREADS>(my_items) >= slots_h) {
    __syncthreads();
    return INT_MAX;
  }
  const int cap_h = p.prefill_piece_cap / p.Hkv;  // partial slots of one head
  const int64_t T64 = (total + slots_h - 1) / slots_h;
  int T = T64 < kSplitMinTiles ? kSplitMinTiles : (T64 > INT_MAX / 2 ? INT_MAX / 2 : (int)T64);
  int64_t my_split = 0;
  for (int s = t; s < p.num_seqs; s += THREADS) {
    int prior, q;
    const int nt = seq_tiles(s, prior, q);
    for (int mt = 0; mt < nt; ++mt) {
      const int n = plan_pieces(item_tiles(prior, q, mt), T);
      if (n > 1) my_split += n;
    }
  }
  if (plan_block_sum<THREADS>(my_split) > cap_h) T *= 2;
  for (int i = t; i < kPlanBins; i += THREADS) bins[i] = 0;
  __syncthreads();
  for (int s = t; s < p.num_seqs; s += THREADS) {
    int prior, q;
    const int nt = seq_tiles(s, prior, q);
    for (int mt = 0; mt < nt; ++mt) {
      const int tiles = item_tiles(prior, q, mt), n = plan_pieces(tiles, T);
      atomicAdd(&bins[bucket(plan_piece_tiles(tiles, n))], n);
    }
  }
  __syncthreads();
  return T;
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
// entries of one bucket in any order.
// bins: kPlanBins ints of LDS; wave_tot: THREADS / 64 ints of LDS.
template <int THREADS>
__device__ void plan_prefill_items(const AttnParams& p, int* bins, int* wave_tot) {
  static_assert(kPlanBins % THREADS == 0, "each thread owns whole bins");
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  const int rows_per_tile = kPrefillPairs / (p.Hq / p.Hkv);
  const int max_len = p.max_blocks * p.bs;
  const int min_rows = p.decode_max_q;
  const int bin_shift = p.plan_bin_shift;
  __shared__ int any_long;                       // some item has more than kSplitMinTiles tiles
  __shared__ int slot_next;                      // partial slots handed out so far (per head)
  for (int i = t; i < kPlanBins; i += THREADS) bins[i] = 0;
  if (t == 0) { any_long = 0; slot_next = 0; }
  __syncthreads();
  auto seq_tiles = [&](int s, int& prior, int& q) -> int {   // row tiles of sequence s
    q = p.qsl[s + 1] - p.qsl[s];
    prior = min(p.seq_lens[s], max_len) - q;
    return q > min_rows ? (q + rows_per_tile - 1) / rows_per_tile : 0;
  };
  // this thread's first sequence is read once and kept in registers for every pass
  int prior0 = 0, q0 = 0, nt0 = 0;
  if (t < p.num_seqs) nt0 = seq_tiles(t, prior0, q0);
  auto seq_of = [&](int s, int& prior, int& q) -> int {
    if (s == t) { prior = prior0; q = q0; return nt0; }
    return seq_tiles(s, prior, q);
  };
  auto item_tiles = [&](int prior, int q, int mt) -> int {   // key tiles of row tile mt
    const int key_end = prior + min((mt + 1) * rows_per_tile, q);
    return (max(key_end, 1) + 63) / 64;
  };
  // bucket of an entry of `tiles` tiles: longest first
  auto bucket = [&](int tiles) { return kPlanBins - 1 - min(tiles >> bin_shift, kPlanBins - 1); };
  // pass 1: the items' buckets, whether any could be split
  for (int s = t; s < p.num_seqs; s += THREADS) {
    int prior, q;
    const int nt = seq_of(s, prior, q);
    for (int mt = 0; mt < nt; ++mt) {
      const int tiles = item_tiles(prior, q, mt);
      atomicAdd(&bins[bucket(tiles)], 1);
      if (tiles > kSplitMinTiles) any_long = 1;
    }
  }
  __syncthreads();
  // the split length T (no item is split when none is longer than kSplitMinTiles)
  const int T = any_long ? plan_split_length<THREADS>(p, bins) : INT_MAX;
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
  // pass 2: the entries; a split item takes n partial slots and clears its counters.  A call
  // with nothing to split takes a copy of the loop with one entry per item (the common case,
  // kept as short as it was before items could be split).
  if (T == INT_MAX) {
    for (int s = t; s < p.num_seqs; s += THREADS) {
      int prior, q;
      const int nt = seq_of(s, prior, q);
      for (int mt = 0; mt < nt; ++mt) {
        const int pos = atomicAdd(&bins[bucket(item_tiles(prior, q, mt))], 1);
        if (pos < p.plan_capacity) p.plan_items[pos] = make_int4(s, mt, 1 << 16, 0);
      }
    }
  } else {
  for (int s = t; s < p.num_seqs; s += THREADS) {
    int prior, q;
    const int nt = seq_of(s, prior, q);
    for (int mt = 0; mt < nt; ++mt) {
      const int tiles = item_tiles(prior, q, mt), n = plan_pieces(tiles, T);
      const int b = bucket(plan_piece_tiles(tiles, n));
      int slot0 = 0;
      if (n > 1) {
        slot0 = atomicAdd(&slot_next, n);        // below the slots of one head by the choice of T
        for (int h = 0; h < p.Hkv; ++h) p.plan_split_ctr[(size_t)slot0 * p.Hkv + h] = 0;
      }
      const int pos = atomicAdd(&bins[b], n);    // the item's pieces side by side in their bucket
      for (int j = 0; j < n; ++j)
        if (pos + j < p.plan_capacity) p.plan_items[pos + j] = make_int4(s, mt, j | (n << 16), slot0);
    }
  }
  }
  if (t == 0) *p.plan_count = min(total_entries, p.plan_capacity);
}

}  // namespace pkv
