/*
 * pagedkv.h -- C ABI of the paged GQA attention library for AMD Instinct MI355X (gfx950).
 *
 * A continuously batched set of sequences keeps its keys and values in a
 * shared pool of fixed-size blocks; each sequence owns a block table that
 * maps its logical block i to a physical block of the pool.  Sources (web
 * pages, cited by title and section):
 *
 *   [TGI]   "Text Generation Inference: Hugging Face's production-grade LLM
 *           inference server" -- "The Investigation" (Finding 2: logical blocks
 *           mapped to physical blocks through a per-sequence block table),
 *           "Under the Hood: PagedAttention" (block table, shared pool, append
 *           of a new token's K/V, gather of K/V tiles through the table),
 *           "Under the Hood: Flash Attention" (exact softmax attention computed
 *           tile by tile with a running max and sum), "Advanced Pattern:
 *           Chunked Prefill" (prompt chunks interleaved with decode rows),
 *           "Production Pattern: KV Cache Math" (bytes per token).
 *   [SPEED] "How to Speed Up LLM Inference: KV Cache to Production Serving" --
 *           "The KV cache: the memory problem that runs the show" (16-token
 *           blocks, GQA, bytes-per-token formula).
 *   [LIFE]  "The inference request lifecycle" -- "KV cache grows with the sum
 *           of cached tokens" (formula; GQA shares K/V heads).
 *   [V3]    pyshine walkthrough of text-generation-inference v3 -- "Inside the
 *           batching task" (every forward has at least one fresh position),
 *           "On the wire" paragraph of "The radix prefix cache" (the scheduler
 *           ships block tables, not KV payloads).
 *
 * Common conventions
 *   bf16      IEEE-754 binary16 "brain float" bit patterns, 2 bytes each.
 *   Pools     k_cache and v_cache are separate device arrays of shape
 *             [num_blocks, block_size, num_kv_heads, head_dim], bf16, dense
 *             row-major.  A slot is block * block_size + offset; slot s's
 *             head-h row starts at element (s * num_kv_heads + h) * head_dim.
 *   GQA       num_q_heads is a multiple of num_kv_heads; query head g reads
 *             KV head g / (num_q_heads / num_kv_heads) (contiguous groups).
 *   Pointers  Arguments marked "device" are device pointers (hipMalloc'd or
 *             equivalent) on the current HIP device; all other arguments are
 *             host values.  The caller owns every buffer; the library never
 *             allocates or frees device memory, never synchronises the
 *             stream and never copies device data to the host.
 *   Streams   `stream` is a hipStream_t (NULL = the null stream).  Work is
 *             enqueued in call order; returning PKV_OK means enqueued, not
 *             finished.
 *   Errors    Argument checks run on the host before any HIP call.  On any
 *             error nothing is enqueued.  Device-side metadata (slots, table
 *             entries, lengths) is the caller's contract: kernels clamp or
 *             skip out-of-range entries instead of touching memory outside
 *             the pools, but the results for such inputs are unspecified.
 */
#ifndef PAGEDKV_H_
#define PAGEDKV_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define PKV_API __attribute__((visibility("default")))
#else
#define PKV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define PKV_OK            0   /* enqueued (or nothing to do)                        */
#define PKV_EINVAL       (-1) /* null pointer, negative size, inconsistent shapes  */
#define PKV_EUNSUPPORTED (-2) /* a shape the kernels are not built for             */
#define PKV_EWORKSPACE   (-3) /* workspace too small (see paged_attention)         */
#define PKV_EHIP         (-4) /* a HIP launch reported an error                    */
#define PKV_ENOSPACE     (-5) /* allocator: not enough blocks even after eviction   */
#define PKV_ESCRATCH     (-6) /* the shape needs more than the static scratch holds */

/*
 * kv_bytes_per_token -- bytes of K plus V that one token occupies in the cache.
 *
 * [TGI] "Production Pattern: KV Cache Math", [SPEED] "The KV cache..." and
 * [LIFE] "KV cache grows with the sum of cached tokens": 2 (one K, one V) x
 * layers x KV heads x head dim x bytes per element.  Pure host integer
 * arithmetic in 64 bits; no HIP call.
 *
 * Returns the byte count, or -1 if any argument is <= 0 or the product does
 * not fit in int64.
 */
PKV_API int64_t kv_bytes_per_token(int64_t num_layers, int64_t num_kv_heads, int64_t head_dim,
                           int64_t dtype_bytes);

/*
 * kv_append -- scatter this step's new K and V rows into their pool slots.
 *
 * [TGI] "Under the Hood: PagedAttention": a generated token's K/V pair is
 * appended at its sequence's next position, in the physical block the block
 * table maps that position to (the caller computes slot_mapping from the
 * tables).  For every i < num_tokens with slot_mapping[i] >= 0:
 *     k_cache row (slot_mapping[i], h) = k_new row (i, h)   for every KV head h
 *     v_cache row (slot_mapping[i], h) = v_new row (i, h)
 * as an exact copy of the bf16 bits.  slot_mapping[i] < 0 marks a padding row
 * and is skipped; a slot >= num_blocks * block_size is skipped as well
 * (caller error; never written).
 *
 *   k_new, v_new   device, bf16 [num_tokens, num_kv_heads, head_dim], read only.
 *   slot_mapping   device, int64 [num_tokens].
 *   num_tokens     >= 0; 0 enqueues nothing and returns PKV_OK (pointers may
 *                  then be NULL).
 *   k_cache, v_cache  device, bf16 pools (see conventions), written in place.
 *   num_blocks, block_size, num_kv_heads, head_dim   pool shape; > 0.
 *   head_dim       a multiple of 8 (16-byte rows chunks); 64 and 128 are tuned.
 *   stream         hipStream_t.
 *
 * Contract: slots are unique within one call (otherwise which row lands is
 * unspecified) and do not target a block mapped by several sequences
 * (shared prefix blocks are copied before a write, [TGI] "Prefix sharing").
 * Enqueue the append before the attention call that reads those tokens.
 * Returns PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED or PKV_EHIP.
 */
PKV_API int kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
              int64_t num_tokens, void* k_cache, void* v_cache, int64_t num_blocks,
              int32_t block_size, int32_t num_kv_heads, int32_t head_dim, void* stream);

/*
 * paged_attention -- causal GQA attention of a mixed batch of decode rows and
 * chunked-prefill rows over the paged cache.
 *
 * Sequence s has seq_lens[s] = L tokens (this step's appended tokens
 * included) and q_s = query_start_loc[s+1] - query_start_loc[s] query rows,
 * which are its last q_s tokens ([TGI] "Advanced Pattern: Chunked Prefill":
 * a chunk continues an already-cached prefix; a decode row is q_s = 1).  Row
 * j of s (global row query_start_loc[s] + j) sits at position p = L - q_s + j
 * and, for every query head g, computes
 *     out[row, g, :] = sum_{t<=p} softmax_t(scale * <q[row, g, :], K_t>) V_t
 * where K_t, V_t are the rows of KV head g / (Hq/Hkv) at position t, found at
 * block block_tables[s, t / block_size], offset t % block_size
 * ([TGI] "Under the Hood: PagedAttention" / "Under the Hood: Flash
 * Attention": exact softmax attention, never materialising the score matrix).
 * Rows of sequences with q_s <= 16 / (num_q_heads / num_kv_heads) -- decode
 * rows and short chunks such as speculative-decoding verification -- share one
 * K/V read per sequence and KV head through split-K with a log-sum-exp merge;
 * longer chunks (chunked prefill) use tiled bf16 matrix-core products, and
 * when a call has too few chunk tiles to occupy the device (a chunk over a
 * long prefix) their long key ranges are cut into pieces whose partial
 * results are merged the same way.  Both accumulate in fp32.  out is rounded to bf16
 * (nearest-even).  Positions >= L and unreferenced blocks are never read into
 * the result (they may hold any bits, NaN included).
 * Shared prefixes ([TGI] "Under the Hood: PagedAttention", prefix sharing):
 * when decode sequences with one row each have block tables that begin with
 * the same physical blocks, the library finds them from the tables (batches
 * of up to 1024 sequences at head_dim 128 with 8 or more KV heads; fewer
 * with fewer KV heads or at head_dim 64) and reads the common whole 64-token
 * tiles once per 16 query
 * columns instead of once per sequence.  The result is the same attention;
 * only the order in which partial sums are combined differs.
 *
 *   out            device, bf16 [num_q_tokens, num_q_heads, head_dim], written.
 *   q              device, bf16 [num_q_tokens, num_q_heads, head_dim].
 *   k_cache, v_cache  device, bf16 pools.
 *   block_tables   device, int32 [num_seqs, max_blocks_per_seq]; entries for
 *                  logical blocks >= ceil(L / block_size) are never read.
 *   seq_lens       device, int32 [num_seqs].
 *   query_start_loc device, int32 [num_seqs + 1], non-decreasing,
 *                  [0] = 0, [num_seqs] = num_q_tokens.
 *   num_seqs, num_q_tokens   >= 0 (0 enqueues nothing).
 *   max_blocks_per_seq  row length of block_tables; also bounds L:
 *                  every L <= max_blocks_per_seq * block_size.
 *   max_query_len  >= every q_s (host-side bound; sizes the prefill grid and
 *                  the decode-row partials of the workspace).
 *   num_q_heads, num_kv_heads   Hq % Hkv == 0 and Hq/Hkv in {1,2,4,8,16}.
 *   head_dim       64 or 128.
 *   num_blocks, block_size   pool shape; block_size in {8, 16, 32}.
 *   scale          softmax scale applied to <q, k> (e.g. 1/sqrt(head_dim)).
 *   workspace      device scratch for split-K partials, or NULL.
 *   workspace_bytes  in/out.  If workspace == NULL, the required size is
 *                  written to *workspace_bytes and nothing is enqueued.
 *                  Otherwise *workspace_bytes is the size of the buffer the
 *                  caller passes (PKV_EWORKSPACE if smaller than required).
 *                  The size depends only on num_seqs, num_q_heads,
 *                  num_kv_heads, head_dim, max_blocks_per_seq, block_size
 *                  and the current device (its compute-unit count sizes the
 *                  decode partials), not on max_query_len.  The buffer needs
 *                  no initialisation and must not be shared by calls that
 *                  can run concurrently.
 *   stream         hipStream_t.
 *
 * Contract: 1 <= q_s <= L for every sequence with rows (q_s = 0 is allowed
 * and produces nothing); rows of different sequences may appear in any
 * order.  Returns PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EWORKSPACE or
 * PKV_EHIP.
 */
PKV_API int paged_attention(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens,
                    const int32_t* query_start_loc, int32_t num_seqs, int64_t num_q_tokens,
                    int32_t max_blocks_per_seq, int32_t max_query_len, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                    int32_t block_size, float scale, void* workspace, size_t* workspace_bytes,
                    void* stream);

/*
 * paged_attention_append -- kv_append and paged_attention of one step in one
 * call, for the step's new tokens ([TGI] "Under the Hood: PagedAttention":
 * each new token's K/V is stored in its sequence's block before attention
 * reads the sequence; "Advanced Pattern: Kernel Fusion": the per-step cache
 * bookkeeping is worth folding into the kernels that run anyway).
 *
 * The result is exactly that of
 *     kv_append(k_new, v_new, slot_mapping, num_q_tokens, k_cache, v_cache, ...)
 *     paged_attention(out, q, k_cache, v_cache, ...)
 * (pools and out bit for bit) when row i of k_new / v_new is the new token of
 * query row i -- the token at position L - q_s + j of its sequence for global
 * row query_start_loc[s] + j -- and slot_mapping[i] is that position's slot
 * under block_tables.  Decode rows read their new tokens from k_new / v_new
 * directly; every row is stored into the pools within the same call, after
 * the decode rows have read the pools and before the chunked-prefill rows do.
 *
 *   k_new, v_new   device, bf16 [num_q_tokens, num_kv_heads, head_dim].
 *   slot_mapping   device, int64 [num_q_tokens]; slots < 0 or outside the
 *                  pool are not stored (and must then not be read by
 *                  the attention: the contract above requires real slots).
 *   k_cache, v_cache  device, bf16 pools, written in place.
 *   Every other argument, the workspace (same size as paged_attention's) and
 *   the return codes are those of paged_attention.
 */
PKV_API int paged_attention_append(void* out, const void* q, const void* k_new, const void* v_new,
                                   const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                   const int32_t* block_tables, const int32_t* seq_lens,
                                   const int32_t* query_start_loc, int32_t num_seqs, int64_t num_q_tokens,
                                   int32_t max_blocks_per_seq, int32_t max_query_len, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                                   int32_t block_size, float scale, void* workspace, size_t* workspace_bytes,
                                   void* stream);

/*
 * paged_attention_append_noalloc -- paged_attention_append without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * Same arguments (minus workspace / workspace_bytes), same kernels and same
 * result, pools and out bit for bit.  The split-K partials and the prefill
 * work list go to a static device array of the library, PKV_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU, held by each GPU the library runs on until the process
 * ends; its address is looked up once per device on the first call there.
 * The call allocates, frees and clears nothing: the scratch needs no
 * initialisation (every value is written before it is read within a call).
 *
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one GPU (different streams without an ordering between them) race and give
 * unspecified results.  Order them on one stream or with events.
 *
 * Returns what paged_attention_append returns, or PKV_ESCRATCH (nothing
 * enqueued) when the shape needs more scratch than PKV_NOALLOC_SCRATCH_BYTES
 * (paged_attention's workspace query gives the size a shape needs; on a
 * 256-CU device, 64 sequences of up to 4096 tokens with 32 query heads of
 * dimension 128 need about 36 MB, 4 sequences of 131072 tokens with 64 query
 * heads about 35 MB: most of it is the decode partials, sized by the CU count).
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
PKV_API int paged_attention_append_noalloc(void* out, const void* q, const void* k_new, const void* v_new,
                                           const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                           const int32_t* block_tables, const int32_t* seq_lens,
                                           const int32_t* query_start_loc, int32_t num_seqs,
                                           int64_t num_q_tokens, int32_t max_blocks_per_seq,
                                           int32_t max_query_len, int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int64_t num_blocks, int32_t block_size,
                                           float scale, void* stream);

/*
 * 8-bit (FP8 E4M3) cache.
 *
 * [SPEED] "The KV cache: the memory problem that runs the show": quantising the
 * cache itself to FP8 halves the bytes per token; "Quantization: move fewer
 * bytes": values are stored in few bits with a shared scale factor and are
 * dequantised in registers before they are multiplied, so the gain is
 * bandwidth.  [TGI] "Production Pattern: KV Cache Math": one byte per value
 * (kv_bytes_per_token(..., 1)).
 *
 * Format (a reading; the pages name no encoding): E4M3 without infinities --
 * sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
 * holds the subnormals m * 2^-9; S.1111.111 is NaN; largest magnitude 448.
 * Scale (a reading; the pages give no convention): one float per pool, K and
 * V separately, chosen by the caller; a code c in the K pool stands for
 * value(c) * k_scale.  Pools have the bf16 pools' shape [num_blocks,
 * block_size, num_kv_heads, head_dim] with one byte per value.
 */

/*
 * kv_append_fp8 -- quantise this step's new K and V rows into an 8-bit pool.
 *
 * Slot semantics exactly as kv_append.  Every value x of k_new (v_new)
 * becomes the E4M3 code nearest to y = x / k_scale (x / v_scale), y being the
 * correctly rounded float32 quotient; an exact tie takes the code with an even
 * mantissa; |y| >= 448 (and a NaN x) gives the largest finite code of y's
 * sign (saturation).
 *
 *   k_new, v_new   device, bf16 [num_tokens, num_kv_heads, head_dim].
 *   slot_mapping   device, int64 [num_tokens]; < 0 = padding (skipped).
 *   k_cache, v_cache  device, uint8 E4M3 pools, written in place.
 *   head_dim       a multiple of 16 (rows move in 16-byte chunks of codes).
 *   k_scale, v_scale  finite and > 0 (PKV_EINVAL otherwise).
 * Returns PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED or PKV_EHIP.
 */
PKV_API int kv_append_fp8(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                  int64_t num_tokens, void* k_cache, void* v_cache, int64_t num_blocks,
                  int32_t block_size, int32_t num_kv_heads, int32_t head_dim, float k_scale,
                  float v_scale, void* stream);

/*
 * paged_attention_fp8 -- paged_attention over 8-bit pools.
 *
 * Computes, for the same rows and with the same arguments as paged_attention,
 * the softmax attention of the dequantised rows value(code) * k_scale and
 * value(code) * v_scale.  The kernels widen codes exactly to bf16 (every E4M3
 * value is a bf16 value), fold k_scale into the score scale and v_scale into
 * the output; accumulation is fp32 and out is bf16 as for bf16 pools.  The
 * workspace is the one paged_attention needs for the same shapes (query it
 * with workspace == NULL here or there).  head_dim 64 needs block_size 16 or
 * 32 (PKV_EUNSUPPORTED for 8).  k_scale, v_scale finite and > 0.
 * Returns PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EWORKSPACE or PKV_EHIP.
 */
PKV_API int paged_attention_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* seq_lens,
                        const int32_t* query_start_loc, int32_t num_seqs, int64_t num_q_tokens,
                        int32_t max_blocks_per_seq, int32_t max_query_len, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                        int32_t block_size, float scale, float k_scale, float v_scale,
                        void* workspace, size_t* workspace_bytes, void* stream);

/*
 * kv_copy_blocks -- copy whole pool blocks, K and V (copy-on-write).
 *
 * [TGI] "Under the Hood: PagedAttention", "Prefix sharing": when a sequence
 * writes into a block it shares, the block is first copied to a new physical
 * block and the writer's table points there.  For every i < n_pairs with
 * src[i] != dst[i] and both in [0, num_blocks): block dst[i] of k_cache and of
 * v_cache becomes a bit copy of block src[i].  Pairs outside the pool are
 * skipped.  Works for bf16 and 8-bit pools (elem_bytes 2 or 1).
 *
 *   k_cache, v_cache  device pools [num_blocks, block_size, num_kv_heads, head_dim].
 *   src, dst       device, int32 [n_pairs]; the dst blocks are distinct and
 *                  none is a src of the same call (otherwise the result is
 *                  unspecified).
 *   n_pairs        >= 0 (0 enqueues nothing).
 *   block_size * num_kv_heads * head_dim * elem_bytes must be a multiple of 16.
 * Returns PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED or PKV_EHIP.
 */
PKV_API int kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst,
                   int32_t n_pairs, int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, int32_t elem_bytes, void* stream);

/*
 * Host block allocator with a radix prefix cache.
 *
 * [V3] "The radix prefix cache": the scheduler owns a block allocator that
 * keeps block 0 back, a free list, and a compressed radix tree of cached
 * prefixes keyed by token ids at block granularity.  Allocating walks the
 * tree with the prompt, references the deepest matched node before anything
 * can be evicted, and takes fresh blocks for the rest, evicting the least
 * recently used unreferenced prefixes when the free list runs dry; freeing
 * drops the reference and inserts the computed prefix (splitting an edge
 * where tokens diverge), returning blocks that another request cached in the
 * meantime.  [V3] "Inside the batching task": a prompt always keeps one token
 * to compute.  [TGI] "Prefix sharing": shared blocks are copied on write.
 * The tables and slots it returns feed kv_append / paged_attention.
 *
 * Readings (the pages are silent): only whole blocks are cached and matched
 * (at most floor((n_prompt - 1) / block_size) blocks of a prompt); fresh
 * blocks are handed out lowest id first; every allocate, free, growing
 * extend and copying prepare_write advances a clock; eviction removes whole
 * unreferenced leaves, least recently used first, ties to the oldest node; a
 * block returns to the free list when no live allocation and no cached
 * prefix holds it.  Host memory only, no HIP call; not thread-safe (one
 * caller at a time per allocator).  Every call returns PKV_OK, PKV_EINVAL
 * (null handle/pointer, unknown id, argument out of range, output capacity
 * too small -- nothing changed) or PKV_ENOSPACE (nothing changed, except the
 * clock and a tree split that does not change any cached content).
 */
typedef struct pkv_allocator pkv_allocator;

/* num_blocks >= 2 (block 0 is never handed out), block_size >= 1; NULL on error. */
PKV_API pkv_allocator* pkv_allocator_create(int32_t num_blocks, int32_t block_size);
PKV_API void pkv_allocator_destroy(pkv_allocator* a);

/* Blocks for a request with prompt tokens[0..n_tokens) that will hold n_total >= max(1,
 * n_tokens) tokens.  Writes its id, its ceil(n_total / block_size) blocks (cached prefix
 * first) into blocks[0..capacity) with the count in *n_blocks, and in *prefix_len the number
 * of prompt tokens whose K/V is already cached (a multiple of block_size). */
PKV_API int pkv_allocator_allocate(pkv_allocator* a, const int32_t* tokens, int32_t n_tokens,
                           int32_t n_total, int64_t* alloc_id, int32_t* blocks, int32_t capacity,
                           int32_t* n_blocks, int32_t* prefix_len);

/* End an allocation whose K/V now holds tokens[0..n_tokens); its whole blocks are cached.
 * The tokens must be what the blocks hold: a block shared through fork holds the same tokens
 * for every holder (writes go through prepare_write).  Tokens that contradict a shared block's
 * content cache that block under a second prefix (it then counts twice in num_cached; it is
 * still not handed out while any prefix or allocation holds it). */
PKV_API int pkv_allocator_free(pkv_allocator* a, int64_t alloc_id, const int32_t* tokens,
                       int32_t n_tokens);

/* A new allocation sharing the blocks that hold the first n_tokens tokens of alloc_id
 * (blocks may be NULL: only the id and count are returned). */
PKV_API int pkv_allocator_fork(pkv_allocator* a, int64_t alloc_id, int32_t n_tokens, int64_t* new_id,
                       int32_t* blocks, int32_t capacity, int32_t* n_blocks);

/* Grow an allocation to hold n_total tokens (fresh blocks at its end); returns its table. */
PKV_API int pkv_allocator_extend(pkv_allocator* a, int64_t alloc_id, int32_t n_total, int32_t* blocks,
                         int32_t capacity, int32_t* n_blocks);

/* Call before writing token position pos.  If its block is shared, the allocation gets a
 * fresh block instead and *src, *dst name the block copy the caller must make on the
 * device (kv_copy_blocks) before the write; otherwise *src = *dst = -1. */
PKV_API int pkv_allocator_prepare_write(pkv_allocator* a, int64_t alloc_id, int32_t pos, int32_t* src,
                                int32_t* dst);

/* slots[i] = block of position start + i times block_size plus its offset (kv_append's
 * slot_mapping); positions must lie inside the allocation. */
PKV_API int pkv_allocator_slots(pkv_allocator* a, int64_t alloc_id, int32_t start, int32_t count,
                        int64_t* slots);

/* The allocation's block table (a row of paged_attention's block_tables). */
PKV_API int pkv_allocator_table(pkv_allocator* a, int64_t alloc_id, int32_t* blocks, int32_t capacity,
                        int32_t* n_blocks);

/* Free blocks, and blocks held by cached prefixes (-1 for a NULL handle). */
PKV_API int32_t pkv_allocator_num_free(const pkv_allocator* a);
PKV_API int32_t pkv_allocator_num_cached(const pkv_allocator* a);

/*
 * pkv_check_metadata -- checks one step's metadata on the device against the
 * contract of kv_append and paged_attention (a debugging aid; the attention
 * calls themselves never test it).  The relations are those of the block-table
 * scheme ([TGI] "Under the Hood: PagedAttention": logical block i of a
 * sequence lives in the physical block its table names, and a new token is
 * stored at its position's slot) and of chunked prefill ([TGI] "Advanced
 * Pattern: Chunked Prefill": the q_s rows of a sequence of L tokens are its
 * positions L - q_s .. L - 1).
 *
 *   block_tables, seq_lens, query_start_loc, num_seqs, num_q_tokens,
 *   max_blocks_per_seq, max_query_len, num_blocks, block_size
 *                  as in paged_attention (device arrays, host scalars).
 *   slot_mapping   device, int64 [num_q_tokens] -- the slots of this step's
 *                  new tokens, row i being the token of query row i (the
 *                  layout of paged_attention_append) -- or NULL to skip the
 *                  slot checks.
 *   error_word     device int32, written: cleared, then the OR of the flags
 *                  below for every violation found (0: the contract holds).
 *                  Read it after the stream reaches this point.
 *   stream         hipStream_t.
 *
 * Not checked: that slots are distinct within a call and that no slot lies
 * in a block shared with another sequence (both need the whole pool's
 * ownership, which the allocator holds).  Returns PKV_OK, PKV_EINVAL (null
 * error_word or query_start_loc, null tables or lengths with num_seqs > 0,
 * negative sizes, block_size <= 0; nothing enqueued) or PKV_EHIP.
 */
#define PKV_META_QSL         0x01  /* query_start_loc[0] != 0, decreasing, or last != num_q_tokens */
#define PKV_META_QUERY_LEN   0x02  /* some q_s > max_query_len                                  */
#define PKV_META_LENGTH      0x04  /* some L < 0, or a sequence with rows has L < q_s            */
#define PKV_META_TABLE_SPAN  0x08  /* some L > max_blocks_per_seq * block_size                    */
#define PKV_META_TABLE_ENTRY 0x10  /* a needed table entry (block < ceil(L / bs)) outside [0, NB) */
#define PKV_META_SLOT_RANGE  0x20  /* a row's slot >= num_blocks * block_size                      */
#define PKV_META_SLOT_TABLE  0x40  /* a row's slot is not its position's slot under the table      */
PKV_API int pkv_check_metadata(const int32_t* block_tables, const int32_t* seq_lens,
                               const int32_t* query_start_loc, int32_t num_seqs, int64_t num_q_tokens,
                               int32_t max_blocks_per_seq, int32_t max_query_len,
                               const int64_t* slot_mapping, int64_t num_blocks, int32_t block_size,
                               int32_t* error_word, void* stream);

/* Human-readable name of a status code (static string). */
PKV_API const char* pkv_status_string(int status);

/*
 * Measurement helpers (not part of the attention path): the device rates the
 * attention kernels' figures are read against, measured on the GPU at hand.
 *
 * pkv_peak_read -- one streaming read of `bytes` (a multiple of 16) at `buf`
 * (device, 16-byte aligned) with the non-temporal loads the decode kernel
 * uses; `sink` is a device word that is never written in practice.  Time the
 * call with events on `stream`: bytes / time is the read rate.
 *
 * pkv_peak_mfma_bf16 -- every wave of a two-waves-per-SIMD grid issues
 * `iterations` x 8 independent v_mfma_f32_32x32x16_bf16 on register operands;
 * *flops receives the floating-point operations the launch performs.
 *
 * Both return PKV_OK, PKV_EINVAL (bad pointer, size or count; nothing
 * enqueued) or PKV_EHIP.
 */
PKV_API int pkv_peak_read(const void* buf, int64_t bytes, void* sink, void* stream);
PKV_API int pkv_peak_mfma_bf16(int64_t iterations, void* sink, int64_t* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H_ */
