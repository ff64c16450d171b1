// Prefill work list of one attention call, built by one workgroup of the plan launch
// (which runs before the decode, merge and prefill kernels on the same stream).
#pragma once

#include "common.h"
#include "kernels.h"

namespace pkv {

// Buckets of the counting sort: item tile counts are shifted right by plan_bin_shift so
// that the largest fits.
constexpr int kPlanBins = kPlanBinsHost;

// Lists the prefill work items (sequence, row tile) of one call, longest first.  A
// sequence with q_s > decode_max_q rows (fewer are computed as decode rows) has
// ceil(q_s / rows_per_tile) row tiles; row tile mt needs the keys before position
// L - q_s + min((mt + 1) rows_per_tile, q_s), i.e. that many keys / 64 tiles of work.
// Workgroups start in id order as earlier ones finish, so listing the items by
// decreasing work is the longest-processing-time-first schedule: the long items (late
// row tiles of long prefixes) are not left to start last.  A counting sort over the
// items' tile counts; items of one bucket in any order.  The first round of sequences'
// lengths is kept in registers between the two passes.
// bins: kPlanBins ints of LDS; wave_tot: THREADS / 64 ints of LDS.
template <int THREADS>
__device__ void plan_prefill_items(const AttnParams& p, int* bins, int* wave_tot) {
  static_assert(kPlanBins % THREADS == 0, "each thread owns whole bins");
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  const int rows_per_tile = kPrefillPairs / (p.Hq / p.Hkv);
  const int max_len = p.max_blocks * p.bs;
  const int min_rows = p.decode_max_q;
  const int bin_shift = p.plan_bin_shift;
  for (int i = t; i < kPlanBins; i += THREADS) bins[i] = 0;
  __syncthreads();
  // bucket of row tile mt of a sequence (q rows after prior cached keys): longest first
  auto bucket = [&](int prior, int q, int mt) {
    const int key_end = prior + min((mt + 1) * rows_per_tile, q);
    const int tiles = (max(key_end, 1) + 63) / 64;
    return kPlanBins - 1 - min(tiles >> bin_shift, kPlanBins - 1);
  };
  auto seq_tiles = [&](int s, int& prior, int& q) -> int {   // row tiles of sequence s
    q = p.qsl[s + 1] - p.qsl[s];
    prior = min(p.seq_lens[s], max_len) - q;
    return q > min_rows ? (q + rows_per_tile - 1) / rows_per_tile : 0;
  };
  int prior0 = 0, q0 = 0, nt0 = 0;               // this thread's first sequence, reused below
  for (int s = t; s < p.num_seqs; s += THREADS) {
    int prior, q;
    const int nt = seq_tiles(s, prior, q);
    if (s == t) { prior0 = prior; q0 = q; nt0 = nt; }
    for (int mt = 0; mt < nt; ++mt) atomicAdd(&bins[bucket(prior, q, mt)], 1);
  }
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
  int total = 0;
  for (int i = 0; i < THREADS / kWave; ++i) total += wave_tot[i];
  for (int i = 0; i < PER; ++i) {
    const int c = bins[PER * t + i];
    bins[PER * t + i] = run;
    run += c;
  }
  __syncthreads();
  for (int s = t; s < p.num_seqs; s += THREADS) {
    int prior = prior0, q = q0, nt = nt0;
    if (s != t) nt = seq_tiles(s, prior, q);
    for (int mt = 0; mt < nt; ++mt) {
      const int pos = atomicAdd(&bins[bucket(prior, q, mt)], 1);
      if (pos < p.plan_capacity) p.plan_items[pos] = make_int2(s, mt);
    }
  }
  if (t == 0) *p.plan_count = min(total, p.plan_capacity);
}

}  // namespace pkv
