// C ABI of the library (declared in include/pagedkv.h): host-side argument
// checks, workspace sizing and kernel dispatch.  No HIP call is made before
// every argument has been validated.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "kernels.h"
#include "pagedkv.h"

namespace {

constexpr int kMinShareTokens = 512;   // smallest key range a decode wave takes (a multiple of 64)
constexpr int kDecodeWavesPerCU = 8;   // resident decode waves per compute unit (2 per SIMD)

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WsLayout {
  int64_t max_splits;
  int64_t plan_capacity;
  int64_t piece_cap;
  size_t ctr_off;
  int64_t share_seqs, mem_rows0;
  size_t o_off, m_off, l_off, nparts_off, memrec_off, count_off, items_off, total;
};

// The largest number of sequences a call may have for its decode rows to be checked for shared
// prefix blocks: each decode wave hashes the sequences' first blocks in its own tile buffer (at
// most a quarter full), a workgroup builds the plan in its tile buffers (2 hash slots and 8 ints
// per sequence, plus a few per thread), and keeps it after them in LDS, where the (8 / group)
// workgroups a compute unit holds must still fit in its 160 KiB.
int share_cap(int D, int group) {
  const int tile_ints = 64 * (D / 8) * 4;        // ints of one wave's tile buffer
  int cap = std::min(pkv::kShareMaxSeqs, tile_ints / 4);
  while (cap > 0 && 12 * cap + group * 64 + 16 > group * tile_ints) cap /= 2;
  while (cap > 0 && (size_t)(8 / group) * ((size_t)group * tile_ints + pkv::share_plan_ints(cap)) * 4 >
                        (size_t)160 * 1024)
    cap /= 2;
  return cap;
}

// Rows per sequence that are computed as decode rows: q_s x G (row, head) columns fill
// at most the 16 columns of the decode kernel's score product.
int decode_rows(int Hq, int Hkv, int max_query_len) {
  const int by_columns = 16 / (Hq / Hkv);
  return std::max(1, std::min(by_columns, max_query_len));
}

// Decode waves of one call: the device's compute units times the resident waves per unit,
// looked up once per device.
int decode_waves_for_current_device() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
  if (dev >= 0) {
    const int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const int waves = cus * kDecodeWavesPerCU;
  if (dev >= 0) cached[dev].store(waves, std::memory_order_relaxed);
  return waves;
}

// Split-K partials of decode rows and the pieces' records, then the prefill planner's
// count and work list.  A decode workgroup leaves at most two partial pieces that do not
// cover their segment (the first and the last of its share), each a row of 16 columns per
// wave: decode_waves x 2 x 16 rows of D + 2 floats whatever the batch.  Calls checked for
// shared prefixes (share_seqs = num_seqs) add two rows per (sequence, query head) and a
// record per sequence.  A decode wave's share is at least kMinShareTokens keys, so a
// (sequence, head) of at most max_blocks * bs keys is cut into at most
// ceil(max_tokens / kMinShareTokens) + 1 pieces (max_splits; it picks the merge form).
WsLayout workspace_layout(int num_seqs, int Hq, int Hkv, int D, int max_blocks, int bs, int decode_waves,
                          int group) {
  WsLayout w{};
  const int64_t max_tokens = (int64_t)max_blocks * bs;
  w.max_splits = (max_tokens + kMinShareTokens - 1) / kMinShareTokens + 1;
  const int rows = pkv::kPrefillPairs / (Hq / Hkv);
  w.piece_cap = (int64_t)decode_waves * 2 * 16 / pkv::kPrefillPairs;   // split prefill items reuse the decode partial rows
  w.plan_capacity = (int64_t)num_seqs * ((max_tokens + rows - 1) / rows) + w.piece_cap;
  w.share_seqs = num_seqs <= share_cap(D, group) ? num_seqs : 0;
  w.mem_rows0 = (int64_t)decode_waves * 2 * 16;
  const size_t prows = (size_t)w.mem_rows0 + 2 * (size_t)w.share_seqs * Hq;
  const size_t nseg = (size_t)num_seqs + (size_t)w.share_seqs;
  w.o_off = 0;
  w.m_off = round_up(prows * D * sizeof(float), 256);
  w.l_off = w.m_off + round_up(prows * sizeof(float), 256);
  w.nparts_off = w.l_off + round_up(prows * sizeof(float), 256);
  w.memrec_off = w.nparts_off + round_up(nseg * Hkv * 2 * sizeof(int), 256);
  w.count_off = w.memrec_off + round_up((size_t)w.share_seqs * 2 * sizeof(int), 256);
  w.ctr_off = w.count_off + 256;
  w.items_off = w.ctr_off + round_up((size_t)w.piece_cap * sizeof(int), 256);
  w.total = w.items_off + round_up((size_t)w.plan_capacity * 16, 256);
  return w;
}

// KV heads a decode workgroup takes together: the largest power of two <= 8 dividing Hkv.
int decode_group_for(int Hkv) {
  int g = 1;
  while (g < pkv::kMaxDecodeGroup && Hkv % (2 * g) == 0) g *= 2;
  return g;
}

// Static scratch of paged_attention_append_noalloc: the workspace of one call, in a device
// array of the library (each GPU the library runs on holds its own copy until the process
// ends).  In host code the array's name is only a stand-in for the symbol, never a device
// address: the address is looked up per device with hipGetSymbolAddress, with that device
// current, on its first call, and only that pointer is handed to the kernels.
constexpr size_t kNoallocScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
__device__ __attribute__((aligned(256))) char noalloc_scratch[kNoallocScratchBytes];

void* noalloc_scratch_for_current_device() {
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch)) != hipSuccess || !p) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

}  // namespace

extern "C" {

int64_t kv_bytes_per_token(int64_t num_layers, int64_t num_kv_heads, int64_t head_dim,
                           int64_t dtype_bytes) {
  if (num_layers <= 0 || num_kv_heads <= 0 || head_dim <= 0 || dtype_bytes <= 0) return -1;
  int64_t r = 2;
  const int64_t f[4] = {num_layers, num_kv_heads, head_dim, dtype_bytes};
  for (int i = 0; i < 4; ++i) {
    if (r > INT64_MAX / f[i]) return -1;
    r *= f[i];
  }
  return r;
}

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EUNSUPPORTED: return "unsupported shape";
    case PKV_EWORKSPACE: return "workspace too small";
    case PKV_EHIP: return "HIP launch error";
    case PKV_ENOSPACE: return "no free blocks";
    case PKV_ESCRATCH: return "shape needs more than the static scratch";
  }
  return "unknown status";
}

int kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping, int64_t num_tokens,
              void* k_cache, void* v_cache, int64_t num_blocks, int32_t block_size,
              int32_t num_kv_heads, int32_t head_dim, void* stream) {
  if (num_tokens < 0 || num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return PKV_EINVAL;
  if (head_dim % 8 != 0) return PKV_EUNSUPPORTED;   // rows move in 16-byte chunks
  if (num_blocks > INT64_MAX / block_size) return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;               // empty inputs may carry null pointers
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PKV_EINVAL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8))
    return PKV_EINVAL;
  const int row_chunks = num_kv_heads * head_dim / 8;
  hipError_t e = pkv::launch_append(k_new, v_new, slot_mapping, num_tokens, k_cache, v_cache,
                                    num_blocks * block_size, row_chunks, (hipStream_t)stream);
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}

int kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst, int32_t n_pairs,
                   int64_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                   int32_t elem_bytes, void* stream) {
  if (n_pairs < 0 || num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      (elem_bytes != 1 && elem_bytes != 2))
    return PKV_EINVAL;
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * elem_bytes;
  if (block_bytes % 16 != 0) return PKV_EUNSUPPORTED;
  if (n_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src || !dst) return PKV_EINVAL;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(src, 4) || !aligned(dst, 4)) return PKV_EINVAL;
  hipError_t e = pkv::launch_copy_blocks(k_cache, v_cache, src, dst, n_pairs, num_blocks, block_bytes / 16,
                                         (hipStream_t)stream);
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}

int kv_append_fp8(const void* k_new, const void* v_new, const int64_t* slot_mapping, int64_t num_tokens,
                  void* k_cache, void* v_cache, int64_t num_blocks, int32_t block_size,
                  int32_t num_kv_heads, int32_t head_dim, float k_scale, float v_scale, void* stream) {
  if (num_tokens < 0 || num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return PKV_EINVAL;
  if (!(isfinite(k_scale) && k_scale > 0.f && isfinite(v_scale) && v_scale > 0.f)) return PKV_EINVAL;
  if (head_dim % 16 != 0) return PKV_EUNSUPPORTED;  // rows move in 16-byte chunks of codes
  if (num_blocks > INT64_MAX / block_size) return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PKV_EINVAL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8))
    return PKV_EINVAL;
  const int row_chunks16 = num_kv_heads * head_dim / 16;
  hipError_t e = pkv::launch_append_fp8(k_new, v_new, slot_mapping, num_tokens, k_cache, v_cache,
                                        num_blocks * block_size, row_chunks16, k_scale, v_scale,
                                        (hipStream_t)stream);
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // extern "C"

namespace {

// paged_attention and paged_attention_fp8: argument checks, workspace, launches.
int attention_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_tables, const int32_t* seq_lens, const int32_t* query_start_loc,
                   int32_t num_seqs, int64_t num_q_tokens, int32_t max_blocks_per_seq, int32_t max_query_len,
                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                   int32_t block_size, float scale, bool fp8, float k_scale, float v_scale, void* workspace,
                   size_t* workspace_bytes, void* stream, const void* k_new = nullptr,
                   const void* v_new = nullptr, const int64_t* slot_mapping = nullptr, bool fused = false) {
  if (!workspace_bytes) return PKV_EINVAL;
  if (fp8 && !(isfinite(k_scale) && k_scale > 0.f && isfinite(v_scale) && v_scale > 0.f)) return PKV_EINVAL;
  if (num_seqs < 0 || num_q_tokens < 0 || max_blocks_per_seq < 1 || max_query_len < 0 ||
      num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0 || block_size <= 0)
    return PKV_EINVAL;
  if (num_q_heads % num_kv_heads != 0) return PKV_EINVAL;
  if (!isfinite(scale)) return PKV_EINVAL;
  const int G = num_q_heads / num_kv_heads;
  if (!pkv::decode_supported(head_dim, G, block_size, fp8) || !pkv::prefill_supported(head_dim, G, block_size, fp8))
    return PKV_EUNSUPPORTED;
  if (num_seqs > 65535 || num_q_heads > 65535) return PKV_EUNSUPPORTED;   // 16-bit sequence and head counts
  const int decode_waves = decode_waves_for_current_device();
  const int group = decode_group_for(num_kv_heads);
  const WsLayout ws = workspace_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                                       block_size, decode_waves, group);
  if (ws.max_splits > 65535 || ws.plan_capacity > INT32_MAX) return PKV_EUNSUPPORTED;
  // decode work units (sequence, KV head, 64-token tile) are counted in 32 bits
  if ((int64_t)num_seqs * num_kv_heads * (((int64_t)max_blocks_per_seq * block_size + 63) / 64) > INT32_MAX)
    return PKV_EUNSUPPORTED;
  if (!workspace) {
    *workspace_bytes = ws.total;
    return PKV_OK;
  }
  if (*workspace_bytes < ws.total) return PKV_EWORKSPACE;
  if (!aligned(workspace, 256)) return PKV_EINVAL;
  if (num_seqs == 0 || num_q_tokens == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens || !query_start_loc)
    return PKV_EINVAL;
  if (max_query_len < 1) return PKV_EINVAL;   // rows exist, so some sequence has q_s >= 1
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return PKV_EINVAL;
  if (fused && (!k_new || !v_new || !slot_mapping || !aligned(k_new, 16) || !aligned(v_new, 16) ||
                !aligned(slot_mapping, 8)))
    return PKV_EINVAL;
  if (fused && num_blocks > INT64_MAX / block_size) return PKV_EINVAL;

  pkv::AttnParams p{};
  p.out = (uint16_t*)out;
  p.q = (const uint16_t*)q;
  p.k_cache = (const char*)k_cache;
  p.v_cache = (const char*)v_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.qsl = query_start_loc;
  p.num_seqs = num_seqs;
  p.num_q_tokens = num_q_tokens;
  p.num_blocks = num_blocks;
  p.max_blocks = max_blocks_per_seq;
  p.max_query_len = max_query_len;
  p.Hq = num_q_heads;
  p.Hkv = num_kv_heads;
  p.D = head_dim;
  p.bs = block_size;
  p.scale_log2 = scale * 1.4426950408889634f;
  if (fp8) p.scale_log2 *= k_scale;               // scores of codes, times the K scale
  p.v_scale = fp8 ? v_scale : 1.f;
  if (fused) {
    p.k_new = (const uint16_t*)k_new;
    p.v_new = (const uint16_t*)v_new;
    p.slots = slot_mapping;
    p.k_pool = (uint4*)k_cache;
    p.v_pool = (uint4*)v_cache;
  }
  p.decode_waves = decode_waves;
  // the KV heads a decode workgroup reads together: the largest power of two <= 8 dividing Hkv
  p.decode_group = group;
  p.decode_max_q = decode_rows(num_q_heads, num_kv_heads, max_query_len);
  p.min_share_tiles = kMinShareTokens / 64;
  p.max_splits = ws.max_splits;
  char* wsb = (char*)workspace;
  p.ws_o = (float*)(wsb + ws.o_off);
  p.ws_m = (float*)(wsb + ws.m_off);
  p.ws_l = (float*)(wsb + ws.l_off);
  p.ws_nparts = (int2*)(wsb + ws.nparts_off);
  p.mem_rows0 = ws.mem_rows0;
  p.share_seqs = (int)ws.share_seqs;
  p.share_hash_slots = 2;
  while (p.share_hash_slots < 2 * p.share_seqs) p.share_hash_slots *= 2;
  p.plan_memrec = (int2*)(wsb + ws.memrec_off);
  p.plan_bin_shift = 0;
  while ((((int64_t)max_blocks_per_seq * block_size + 63) / 64 >> p.plan_bin_shift) >= pkv::kPlanBinsHost)
    ++p.plan_bin_shift;
  p.plan_count = (int*)(wsb + ws.count_off);
  p.plan_items = (int4*)(wsb + ws.items_off);
  p.plan_split_ctr = (int*)(wsb + ws.ctr_off);
  p.prefill_piece_cap = (int)ws.piece_cap;
  // prefill workgroups resident at once: two per compute unit (their registers and LDS)
  p.prefill_slots = std::max(1, decode_waves / kDecodeWavesPerCU) * 2;
  p.plan_capacity = (int)ws.plan_capacity;
  {
    // bound on the prefill items of this call: sum over sequences with q_s > 1 of
    // ceil(q_s / rows) <= num_q_tokens / rows + (number of such sequences)
    const int rows = pkv::kPrefillPairs / G;
    // plus the extra pieces of split items (at most the partial slots of one head)
    const int64_t bound = (num_q_tokens + rows - 1) / rows + std::min<int64_t>(num_seqs, num_q_tokens / 2) +
                          ws.piece_cap / num_kv_heads;
    p.plan_stride = (int)std::min<int64_t>(bound, ws.plan_capacity);
  }

  hipStream_t st = (hipStream_t)stream;
  hipError_t e = pkv::launch_decode(p, fp8, st);
  if (e == hipSuccess) e = pkv::launch_merge(p, st);
  if (e == hipSuccess && max_query_len > p.decode_max_q) e = pkv::launch_prefill(p, fp8, st);
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // namespace

extern "C" {

int paged_attention(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens,
                    const int32_t* query_start_loc, int32_t num_seqs, int64_t num_q_tokens,
                    int32_t max_blocks_per_seq, int32_t max_query_len, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t block_size,
                    float scale, void* workspace, size_t* workspace_bytes, void* stream) {
  return attention_impl(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, num_seqs,
                        num_q_tokens, max_blocks_per_seq, max_query_len, num_q_heads, num_kv_heads, head_dim,
                        num_blocks, block_size, scale, false, 1.f, 1.f, workspace, workspace_bytes, stream);
}

int paged_attention_append(void* out, const void* q, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, void* k_cache, void* v_cache,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           const int32_t* query_start_loc, int32_t num_seqs, int64_t num_q_tokens,
                           int32_t max_blocks_per_seq, int32_t max_query_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t block_size,
                           float scale, void* workspace, size_t* workspace_bytes, void* stream) {
  return attention_impl(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, num_seqs,
                        num_q_tokens, max_blocks_per_seq, max_query_len, num_q_heads, num_kv_heads, head_dim,
                        num_blocks, block_size, scale, false, 1.f, 1.f, workspace, workspace_bytes, stream,
                        k_new, v_new, slot_mapping, true);
}

int paged_attention_append_noalloc(void* out, const void* q, const void* k_new, const void* v_new,
                                   const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                   const int32_t* block_tables, const int32_t* seq_lens,
                                   const int32_t* query_start_loc, int32_t num_seqs, int64_t num_q_tokens,
                                   int32_t max_blocks_per_seq, int32_t max_query_len, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                                   int32_t block_size, float scale, void* stream) {
  // the size this shape needs (argument checks of the query form included)
  size_t need = 0;
  int st = attention_impl(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, num_seqs, num_q_tokens,
                          max_blocks_per_seq, max_query_len, num_q_heads, num_kv_heads, head_dim, num_blocks,
                          block_size, scale, false, 1.f, 1.f, nullptr, &need, stream);
  if (st != PKV_OK) return st;
  if (need > kNoallocScratchBytes) return PKV_ESCRATCH;
  void* ws = noalloc_scratch_for_current_device();
  if (!ws) return PKV_EHIP;
  size_t have = kNoallocScratchBytes;
  return attention_impl(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, num_seqs,
                        num_q_tokens, max_blocks_per_seq, max_query_len, num_q_heads, num_kv_heads, head_dim,
                        num_blocks, block_size, scale, false, 1.f, 1.f, ws, &have, stream,
                        k_new, v_new, slot_mapping, true);
}

int paged_attention_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* seq_lens,
                        const int32_t* query_start_loc, int32_t num_seqs, int64_t num_q_tokens,
                        int32_t max_blocks_per_seq, int32_t max_query_len, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t block_size,
                        float scale, float k_scale, float v_scale, void* workspace, size_t* workspace_bytes,
                        void* stream) {
  return attention_impl(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, num_seqs,
                        num_q_tokens, max_blocks_per_seq, max_query_len, num_q_heads, num_kv_heads, head_dim,
                        num_blocks, block_size, scale, true, k_scale, v_scale, workspace, workspace_bytes, stream);
}

}  // extern "C"
