"""Plain float64 reference of the three library calls (test infrastructure only).

Sources (web pages; cited by title and section):
  [TGI]   "Text Generation Inference: Hugging Face's production-grade LLM inference
          server" (nivant-blog) -- sections "Under the Hood: PagedAttention",
          "Under the Hood: Flash Attention", "Advanced Pattern: Chunked Prefill",
          "Production Pattern: KV Cache Math".
  [SPEED] "How to Speed Up LLM Inference: KV Cache to Production Serving"
          (fatherofai) -- section "The KV cache: the memory problem that runs the show".
  [LIFE]  "The inference request lifecycle" (rajjoshi) -- sections "KV cache grows
          with the sum of cached tokens", "Work the GQA number before choosing
          concurrency".
  [V3]    pyshine walkthrough of text-generation-inference v3 -- sections
          "Inside the batching task" (at least one fresh position per forward) and
          "The thin Python shard" (per-block KV cost).

Conventions shared with the library's C header (stated, not imported):
  pools      bf16 bit patterns, shape [num_blocks, block_size, num_kv_heads, head_dim]
  slot       block * block_size + offset
  seq_lens   tokens of each sequence after this step's append
  rows       query rows of sequence s are query_start_loc[s] .. query_start_loc[s+1]-1;
             they are the last q_s tokens of the sequence
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# bf16 decoding (exact)
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the upper half of an IEEE float32; widen the bits and convert exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# kv_bytes_per_token
# ---------------------------------------------------------------------------

def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """Bytes of cached K and V one token occupies across all layers.

    [TGI] "Production Pattern: KV Cache Math" (formula above its table),
    [SPEED] "The KV cache..." (formula block), [LIFE] "KV cache grows with the
    sum of cached tokens": 2 x layers x KV heads x head dim x bytes per value,
    the leading 2 counting one K and one V.  Reading: any argument <= 0 is
    invalid and yields -1 (the pages give no error convention).
    """
    args = (int(num_layers), int(num_kv_heads), int(head_dim), int(dtype_bytes))
    if min(args) <= 0:
        return -1
    L, H, D, B = args
    return 2 * L * H * D * B


# ---------------------------------------------------------------------------
# kv_append
# ---------------------------------------------------------------------------

def kv_append(k_cache, v_cache, k_new, v_new, slot_mapping, block_tables=None, seq_lens=None):
    """Write each new token's K and V rows into its slot; return new pools.

    [TGI] "Under the Hood: PagedAttention": a generated token's K/V pair is
    appended at the next position of its sequence, in the block the block table
    maps that position to.  The slot encodes (block, offset) as
    block * block_size + offset.  The copy is of bf16 bit patterns, unchanged.

    Readings where the pages are silent:
      * slot < 0 marks a padding row and is skipped;
      * a slot outside the pool, or the same slot twice in one call, is an error;
      * with block_tables/seq_lens given, writing into a block that more than
        one sequence maps is an error (shared blocks are copied before a write,
        [TGI] "Prefix sharing" paragraph).
    """
    k_out = np.array(k_cache, dtype=np.uint16, copy=True)
    v_out = np.array(v_cache, dtype=np.uint16, copy=True)
    NB, bs = k_out.shape[0], k_out.shape[1]
    slots = np.asarray(slot_mapping, dtype=np.int64)
    k_new = np.asarray(k_new, dtype=np.uint16)
    v_new = np.asarray(v_new, dtype=np.uint16)
    if k_new.shape[0] != slots.shape[0] or v_new.shape[0] != slots.shape[0]:
        raise ValueError("one slot per new token")
    live = slots[slots >= 0]
    if live.size and live.max() >= NB * bs:
        raise ValueError("slot outside the pool")
    if np.unique(live).size != live.size:
        raise ValueError("duplicate slot in one append")
    if block_tables is not None:
        refs = {}
        bt = np.asarray(block_tables)
        sl = np.asarray(seq_lens)
        for s in range(bt.shape[0]):
            for b in range((int(sl[s]) + bs - 1) // bs):
                refs[int(bt[s, b])] = refs.get(int(bt[s, b]), 0) + 1
        for slot in live:
            if refs.get(int(slot) // bs, 0) > 1:
                raise ValueError("append into a block shared by several sequences")
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        block, offset = int(slot) // bs, int(slot) % bs
        k_out[block, offset] = k_new[i]
        v_out[block, offset] = v_new[i]
    return k_out, v_out


# ---------------------------------------------------------------------------
# paged_attention, one step at a time
# ---------------------------------------------------------------------------

def kv_head_of(g: int, group: int) -> int:
    """GQA: query heads are grouped contiguously, ``group`` = Hq / Hkv per KV head.

    [SPEED] "The KV cache..." item 3 and [LIFE] "KV cache grows with the sum of
    cached tokens": several query heads share one K/V head.  Reading: the
    grouping is contiguous (query head g uses KV head g // group).
    """
    return g // group


def row_position(seq_len: int, q_len: int, j: int) -> int:
    """Absolute position of query row j of a sequence whose last q_len tokens are new.

    [TGI] "Advanced Pattern: Chunked Prefill": a chunk continues a sequence whose
    earlier tokens are already cached; a decode row is the single newest token.
    """
    return seq_len - q_len + j


def gather_tokens(pool: np.ndarray, table_row: np.ndarray, n_tokens: int) -> np.ndarray:
    """Walk one sequence's block table and return its logical rows 0..n_tokens-1.

    [TGI] "Under the Hood: PagedAttention" (the loop over block_table entries
    that fetches each physical block and then each position inside it).
    Returns the pool's element bits (bf16, or FP8 codes), shape [n_tokens, Hkv, D].
    Table entries past the last needed block are never read.
    """
    bs = pool.shape[1]
    out = np.empty((n_tokens,) + pool.shape[2:], dtype=pool.dtype)
    n_blocks = (n_tokens + bs - 1) // bs
    for logical_block in range(n_blocks):
        physical = int(table_row[logical_block])
        first = logical_block * bs
        count = min(bs, n_tokens - first)
        out[first:first + count] = pool[physical, :count]
    return out


def softmax_attend(qh: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """sum_t softmax_t(scale * <q, k_t>) v_t for each query vector in qh.

    [TGI] "Under the Hood: Flash Attention": S = softmax(Q K^T) V; the tiled
    online form computes the same value.  Here: the definition, in float64,
    with the usual max shift (exp(z - max z) / sum, identical in exact math).
    qh [G, D], K [n, D], V [n, D] (all float64) -> [G, D].
    """
    z = scale * (qh @ K.T)                 # [G, n]
    z = z - z.max(axis=1, keepdims=True)
    w = np.exp(z)
    return (w @ V) / w.sum(axis=1, keepdims=True)


def paged_attention(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
                    num_kv_heads: int, scale: float, rows=None) -> np.ndarray:
    """Attention of every query row over its own sequence's cached keys, causally.

    For sequence s with L = seq_lens[s] tokens and q_s = qsl[s+1]-qsl[s] rows,
    row j (global row qsl[s]+j) sits at position p = L - q_s + j and attends the
    keys at positions 0..p, fetched through block_tables[s]; query head g reads
    KV head g // (Hq / Hkv).  The result is the exact softmax attention in
    float64 (bf16 inputs decoded exactly; ``scale`` is the float32 value the
    library receives, widened).

    A row with q_s >= 1 always has p >= 0, so at least one key ([V3] "Inside
    the batching task": a forward always has a fresh position).  Sequences with
    q_s == 0 contribute no rows.  ``rows``: optional iterable of global rows to
    compute (others are left NaN), for sampled checks of large batches.

    q: uint16 bf16 bits [num_q_tokens, Hq, D]; pools: uint16 [NB, bs, Hkv, D];
    block_tables int [num_seqs, max_blocks]; seq_lens int [num_seqs];
    query_start_loc int [num_seqs + 1].  Returns float64 [num_q_tokens, Hq, D].
    """
    q = np.asarray(q, dtype=np.uint16)
    T, Hq, D = q.shape
    Hkv = int(num_kv_heads)
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = Hq // Hkv
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    L_all = np.asarray(seq_lens, dtype=np.int64)
    bt = np.asarray(block_tables)
    scale64 = float(np.float32(scale))
    want = None if rows is None else set(int(r) for r in rows)

    out = np.full((T, Hq, D), np.nan, dtype=np.float64)
    for s in range(L_all.shape[0]):
        a, b = int(qsl[s]), int(qsl[s + 1])
        q_len, L = b - a, int(L_all[s])
        if q_len == 0:
            continue
        if q_len > L:
            raise ValueError("a sequence has more query rows than tokens")
        my_rows = [r for r in range(a, b) if want is None or r in want]
        if not my_rows:
            continue
        K = bf16_bits_to_f64(gather_tokens(k_cache, bt[s], L))   # [L, Hkv, D]
        V = bf16_bits_to_f64(gather_tokens(v_cache, bt[s], L))
        for r in my_rows:
            p = row_position(L, q_len, r - a)
            qr = bf16_bits_to_f64(q[r])                             # [Hq, D]
            for h in range(Hkv):
                heads = [g for g in range(Hq) if kv_head_of(g, group) == h]
                out[r, heads] = softmax_attend(qr[heads], K[:p + 1, h], V[:p + 1, h], scale64)
    return out
