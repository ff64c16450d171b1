// Decode-row bookkeeping shared by the plan, decode and merge kernels.
#pragma once

#include "common.h"
#include "kernels.h"

namespace pkv {

constexpr int kTile = 64;        // keys per decode tile

// First query row, row count, key count and 64-token tiles of sequence s when its rows
// are decode rows -- 1 <= q_s <= decode_max_q, so that its q_s x G (row, head) columns fit
// the 16 columns of the decode kernel's score product -- and no tiles otherwise.
struct SeqInfo {
  int row0, q, len, tiles;
};
// (The three loads are issued together: the checks are combined without short-circuiting.)
__device__ __forceinline__ SeqInfo seq_info(const AttnParams& p, int s) {
  const int row0 = p.qsl[s];
  const int row1 = p.qsl[s + 1];
  const int len = min(p.seq_lens[s], p.max_blocks * p.bs);   // clamp a length the table cannot map
  const int q = row1 - row0;
  const bool bad = (q < 1) | (q > p.decode_max_q) | (row0 < 0) | (row1 > p.num_q_tokens) | (len <= 0);
  if (bad) return SeqInfo{row0, 0, 0, 0};
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

}  // namespace pkv
