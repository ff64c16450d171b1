// Launchers of the gfx950 kernels (internal to the library; the public ABI is include/pagedkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Everything one attention call needs on the device, passed by value to the kernels.
struct AttnParams {
  uint16_t* out;                  // bf16 [num_q_tokens, Hq, D]
  const uint16_t* q;              // bf16 [num_q_tokens, Hq, D]
  const char* k_cache;            // [num_blocks, bs, Hkv, D]: bf16, or E4M3 codes (one byte each)
  const char* v_cache;
  const int32_t* block_tables;    // [num_seqs, max_blocks]
  const int32_t* seq_lens;        // [num_seqs]
  const int32_t* qsl;             // [num_seqs + 1]
  int num_seqs;
  int64_t num_q_tokens;
  int64_t num_blocks;             // pool blocks: table entries outside [0, num_blocks) are skipped
  int max_blocks;
  int max_query_len;
  int Hq, Hkv, D, bs;
  float scale_log2;               // softmax scale * log2(e) (* the K pool scale for E4M3 pools):
                                  // scores live in the exp2 domain
  float v_scale;                  // E4M3 pools: the V pool scale, applied to the output (1 for bf16)
  int decode_waves;               // decode grid: one wave per resident wave slot of the device
  int decode_group;               // decode waves per workgroup: the KV heads taken together (divides Hkv)
  int decode_max_q;               // sequences with 1 <= q_s <= this are decode rows (q_s x G <= 16)
  int min_share_tiles;            // smallest share of 64-token tiles a decode wave takes
  int max_splits;                 // pieces one (sequence, head) can be cut into (picks the merge form)
  // Partials.  Rows [0, decode_waves * 32): the pieces that do not cover their whole segment:
  // a decode workgroup leaves at most two, the first and the last piece of its share (slots 0
  // and 1), each with one row of 16 columns per wave: row ((2 workgroup + slot) * decode_group
  // + wave) * 16 + column.  Then, for sequences of a prefix-sharing group, one row per (sequence,
  // query head) for a whole private segment (row mem_rows0 + s Hq + qh) and one for a whole
  // group segment (row mem_rows0 + (share_seqs + s) Hq + qh).  Segments: sequence s's own
  // tiles (segment s), then the sharing groups' column blocks (segments S, S + 1, ...).
  float* ws_o;                    // [rows, D]  unnormalised partials
  float* ws_m;                    // [rows]     partial max (exp2 domain)
  float* ws_l;                    // [rows]     partial sum of exponentials
  int2* ws_nparts;                // [segments, Hkv]  (slot of the first piece, piece count) of each
                                  // decode segment and KV head; later pieces sit in slot 0 of the
                                  // following workgroups
  int64_t mem_rows0;              // first per-(sequence, head) row
  int share_seqs;                 // sequences checked for shared prefixes: num_seqs, or 0 (no check)
  int share_hash_slots;           // hash table of the sharing plan: a power of two >= 2 share_seqs
  int2* plan_memrec;              // [num_seqs] (group segment S + block, first column) of a member
                                  // of a prefix-sharing group, or (-1, 0); written by the decode
                                  // kernel's workgroup 0 when share_seqs > 0
  // fused append (paged_attention_append; null k_new otherwise): row i of k_new / v_new is the
  // new token of query row i, stored at slot slots[i].  Decode rows read this step's tokens
  // from k_new / v_new; the merge launch scatters every row into the pools afterwards.
  const uint16_t* k_new;          // bf16 [num_q_tokens, Hkv, D]
  const uint16_t* v_new;
  const int64_t* slots;           // [num_q_tokens]; < 0 or >= num_blocks * bs: not stored
  uint4* k_pool;                  // the pools, writable
  uint4* v_pool;
  int merge_blocks;               // merge launch: workgroups that merge (then the append ones)
  int plan_first;                 // merge launch: 1 if its first workgroup plans the prefill items
  int plan_bin_shift;             // prefill planner: tile counts >> this fit its buckets
  int4* plan_items;               // prefill work list, written by the planner: (sequence, row tile,
                                  // piece | pieces << 16, first partial slot of a split item)
  int* plan_count;                // number of valid entries
  int plan_capacity;              // entries the workspace holds
  int plan_stride;                // host bound on the entries of this call (grid = Hkv * stride)
  int prefill_slots;              // prefill workgroups resident at once (two per compute unit)
  int prefill_piece_cap;          // partial slots of split items, all KV heads (rows of ws_o / 128)
  int* plan_split_ctr;            // [prefill_piece_cap] finished pieces per (split item, KV head)
};

// Most KV heads (waves) one decode workgroup takes together.
constexpr int kMaxDecodeGroup = 8;

// Query rows packed into one prefill workgroup (with all G heads of each row).
constexpr int kPrefillPairs = 128;

// Buckets of the prefill planner's counting sort (planner.h).
constexpr int kPlanBinsHost = 4096;

// Prefill items of more than kSplitMinTiles key tiles (64 keys each) may be cut into at most
// kMaxPieces pieces of consecutive tiles when the call has too few items to fill the device.
constexpr int kSplitMinTiles = 64;
constexpr int kMaxPieces = 32;

hipError_t launch_append(const void* k_new, const void* v_new, const int64_t* slots, int64_t num_tokens,
                         void* k_cache, void* v_cache, int64_t num_slots, int row_chunks,
                         hipStream_t stream);
// E4M3 pools: row_chunks16 = 16-byte chunks of codes per pool slot (Hkv * D / 16).
hipError_t launch_append_fp8(const void* k_new, const void* v_new, const int64_t* slots, int64_t num_tokens,
                             void* k_cache, void* v_cache, int64_t num_slots, int row_chunks16,
                             float k_scale, float v_scale, hipStream_t stream);

// Whole-block copies of both pools: pair i copies block src[i] to dst[i] (chunks16 = 16-byte
// chunks per block).
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst, int n_pairs,
                              int64_t num_blocks, int64_t chunks16, hipStream_t stream);

// Sequences of one call up to which decode rows are checked for shared prefix blocks (the
// decode workgroups' LDS then bounds it further).
constexpr int kShareMaxSeqs = 1024;

// Ints of the sharing plan that a decode workgroup keeps in LDS after its tile buffers, for S
// sequences (S rounded up to a multiple of 4, Sr): 4 + Sr + Sr + 2 Sr + (Sr + 4) + 2 Sr.
__host__ __device__ constexpr int share_plan_ints(int S) { return 7 * ((S + 3) & ~3) + 8; }

// fp8: the pools hold E4M3 codes instead of bf16.
bool decode_supported(int D, int G, int bs, bool fp8);
hipError_t launch_decode(const AttnParams& p, bool fp8, hipStream_t stream);
hipError_t launch_merge(const AttnParams& p, hipStream_t stream);

bool prefill_supported(int D, int G, int bs, bool fp8);
hipError_t launch_prefill(const AttnParams& p, bool fp8, hipStream_t stream);

}  // namespace pkv
