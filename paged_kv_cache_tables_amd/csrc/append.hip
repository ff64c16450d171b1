// kv_append: scatter new K/V rows into their pool slots (bit copy).
//
// "Under the Hood: PagedAttention" (Text Generation Inference page): a new
// token's K/V pair is appended at its sequence's next position, inside the
// physical block the sequence's block table maps that position to.  With the
// pool laid out [num_blocks, block_size, kv_heads, head_dim], the flat row of
// slot s is simply s, so the append is a row scatter: every 16-byte chunk of
// new row i goes to chunk c of pool row slot_mapping[i].
#include "common.h"
#include "kernels.h"

namespace pkv {

// One thread per 16-byte chunk of K or V; consecutive threads cover
// consecutive chunks of one row, so loads and stores are fully coalesced.
__global__ __launch_bounds__(256) void append_kernel(const uint4* __restrict__ k_new,
                                                     const uint4* __restrict__ v_new,
                                                     const int64_t* __restrict__ slots,
                                                     int64_t num_tokens, uint4* __restrict__ k_cache,
                                                     uint4* __restrict__ v_cache, int64_t num_slots,
                                                     int row_chunks) {
  const int64_t per_token = 2 * (int64_t)row_chunks;
  const int64_t total = num_tokens * per_token;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = idx / per_token;
    const int rem = (int)(idx - i * per_token);
    const int which = rem >= row_chunks;          // 0 = K, 1 = V
    const int c = rem - which * row_chunks;
    const int64_t slot = slots[i];
    if (slot < 0 || slot >= num_slots) continue;  // padding row, or outside the pool
    const uint4* src = which ? v_new : k_new;
    uint4* dst = which ? v_cache : k_cache;
    dst[slot * row_chunks + c] = src[i * row_chunks + c];
  }
}

hipError_t launch_append(const void* k_new, const void* v_new, const int64_t* slots, int64_t num_tokens,
                         void* k_cache, void* v_cache, int64_t num_slots, int row_chunks,
                         hipStream_t stream) {
  const int64_t total = num_tokens * 2 * (int64_t)row_chunks;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;  // grid-stride loop covers the rest
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     (const uint4*)k_new, (const uint4*)v_new, slots, num_tokens, (uint4*)k_cache,
                     (uint4*)v_cache, num_slots, row_chunks);
  return hipGetLastError();
}

}  // namespace pkv
