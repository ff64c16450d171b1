// Device-side check of one step's metadata against the contract of kv_append and
// paged_attention (a debugging aid, off the attention path): the kernels themselves clamp
// or skip out-of-range entries and never test the contract.
//
// The relations checked are those of the pages' block-table scheme ("Under the Hood:
// PagedAttention" in the Text Generation Inference page: a sequence's logical block i
// lives in the physical block its table names, and a new token is stored at its
// position's slot) and of chunked prefill ("Advanced Pattern: Chunked Prefill": the q_s
// new rows of a sequence of L tokens are its positions L - q_s .. L - 1).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {
namespace {

constexpr int kCheckThreads = 256;

struct CheckArgs {
  const int32_t* bt;
  const int32_t* seq_lens;
  const int32_t* qsl;
  const int64_t* slots;          // may be null
  int32_t num_seqs;
  int64_t num_q_tokens;
  int32_t max_blocks;
  int32_t max_query_len;
  int64_t num_blocks;
  int32_t bs;
  int32_t* err;
};

__global__ void clear_word_kernel(int32_t* w) {
  if (threadIdx.x == 0 && blockIdx.x == 0) w[0] = 0;
}

// One workgroup per sequence (grid-stride): its lengths, the table entries it needs and
// the slots of its rows; every violation found ORs its flag into the error word.
__global__ __launch_bounds__(kCheckThreads) void check_meta_kernel(CheckArgs a) {
  const int tid = threadIdx.x;
  int flags = 0;
  if (blockIdx.x == 0 && tid == 0 && (a.qsl[0] != 0 || a.qsl[a.num_seqs] != a.num_q_tokens))
    flags |= PKV_META_QSL;
  const int64_t slots_total = a.num_blocks * a.bs;
  for (int s = blockIdx.x; s < a.num_seqs; s += gridDim.x) {
    const int64_t r0 = a.qsl[s];
    const int64_t q = (int64_t)a.qsl[s + 1] - r0;
    const int64_t L = a.seq_lens[s];
    if (tid == 0) {
      if (q < 0) flags |= PKV_META_QSL;
      if (q > a.max_query_len) flags |= PKV_META_QUERY_LEN;
      if (L < 0 || (q > 0 && L < q)) flags |= PKV_META_LENGTH;
      if (L > (int64_t)a.max_blocks * a.bs) flags |= PKV_META_TABLE_SPAN;
    }
    const int32_t* row = a.bt + (size_t)s * a.max_blocks;
    const int64_t need = L > 0 ? (L + a.bs - 1) / a.bs : 0;
    const int nb = (int)(need < a.max_blocks ? need : a.max_blocks);
    for (int b = tid; b < nb; b += kCheckThreads) {
      const int32_t e = row[b];
      if (e < 0 || e >= a.num_blocks) flags |= PKV_META_TABLE_ENTRY;
    }
    if (a.slots != nullptr && q > 0) {
      for (int64_t j = tid; j < q; j += kCheckThreads) {
        const int64_t i = r0 + j;
        if (i < 0 || i >= a.num_q_tokens) { flags |= PKV_META_QSL; continue; }
        const int64_t slot = a.slots[i];
        if (slot >= slots_total) flags |= PKV_META_SLOT_RANGE;
        const int64_t pos = L - q + j;
        if (pos < 0 || pos / a.bs >= a.max_blocks) continue;   // flagged above as a length error
        const int64_t want = (int64_t)row[pos / a.bs] * a.bs + pos % a.bs;
        if (slot != want) flags |= PKV_META_SLOT_TABLE;
      }
    }
  }
  if (flags) atomicOr(a.err, flags);
}

}  // namespace
}  // namespace pkv

extern "C" {

int pkv_check_metadata(const int32_t* block_tables, const int32_t* seq_lens, const int32_t* query_start_loc,
                       int32_t num_seqs, int64_t num_q_tokens, int32_t max_blocks_per_seq,
                       int32_t max_query_len, const int64_t* slot_mapping, int64_t num_blocks,
                       int32_t block_size, int32_t* error_word, void* stream) {
  if (!error_word || !query_start_loc || num_seqs < 0 || num_q_tokens < 0 || max_query_len < 0 ||
      num_blocks < 0 || block_size <= 0 || max_blocks_per_seq < 0)
    return PKV_EINVAL;
  if (num_seqs > 0 && (!block_tables || !seq_lens || max_blocks_per_seq < 1)) return PKV_EINVAL;
  pkv::CheckArgs a{block_tables, seq_lens, query_start_loc, num_q_tokens > 0 ? slot_mapping : nullptr,
                   num_seqs, num_q_tokens, max_blocks_per_seq, max_query_len, num_blocks, block_size,
                   error_word};
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(pkv::clear_word_kernel, dim3(1), dim3(64), 0, st, error_word);
  const int grid = num_seqs < 1 ? 1 : (num_seqs < 4096 ? num_seqs : 4096);
  hipLaunchKernelGGL(pkv::check_meta_kernel, dim3(grid), dim3(pkv::kCheckThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // extern "C"
