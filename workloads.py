"""Seeded synthetic inputs for paged GQA attention over block tables.

This module is shared by the tests, the benchmark and the smoke check. It
holds no attention or append arithmetic: it only draws lengths, block
placements and N(0,1) values, rounds the draws to bf16 bit patterns, and lays
the already-cached tokens into a block pool. Both the HIP library and the CPU
oracle consume exactly the arrays it returns.

Workload shapes: a tiny mixed batch, a Llama-3-8B-shaped decode batch, a
70B-class decode batch, a mixed batch with a shared prefix and a long-context
decode batch. The readings taken where the description is silent are stated
next to each generator.

Conventions
  * ``seq_lens[s]`` counts the tokens of sequence s *after* this step's
    ``kv_append``; the last ``q_s`` of them are the new tokens whose K/V arrive
    in ``k_new``/``v_new`` and whose queries are the rows of ``q``.
  * Query rows, new K/V rows and ``slot_mapping`` entries share one ordering:
    row i of ``q`` is new token i.
  * Pool layout is ``[num_blocks, block_size, num_kv_heads, head_dim]`` bf16,
    separate pools for K and V; slot = block * block_size + offset.
  * Every pool slot that holds no cached token is filled with a poison bf16
    pattern (quiet NaN by default).
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)
BF16_PINF = np.uint16(0x7F80)
BF16_NINF = np.uint16(0xFF80)

# SeedSequence stream ids (entropy = [seed, config id, stream, ...])
_S_LENGTHS, _S_PLACEMENT, _S_KV, _S_Q, _S_OUTLIER, _S_SHARE, _S_ORDER, _S_FP8 = range(8)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # uint32 wrap-around can only happen for NaN patterns, which are overridden below
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_QNAN
    return out


_POOL_THREADS = 8


def _par_map(fn, items):
    from concurrent.futures import ThreadPoolExecutor
    items = list(items)
    if len(items) <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(min(_POOL_THREADS, len(items))) as ex:
        return list(ex.map(fn, items))


@dataclass
class Workload:
    """One seeded batch.  The block pools are materialised on first use
    (``k_cache``/``v_cache``): a pool is poison everywhere except the slots of
    already-cached tokens (``cached_slots`` with rows ``cached_k``/``cached_v``)."""
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float                     # a float32 value, carried as a Python float
    q: np.ndarray                    # uint16 [num_q_tokens, Hq, D]   bf16 bits
    k_new: np.ndarray                # uint16 [num_q_tokens, Hkv, D]
    v_new: np.ndarray                # uint16 [num_q_tokens, Hkv, D]
    slot_mapping: np.ndarray         # int64  [num_q_tokens]
    cached_slots: np.ndarray         # int64  [n_cached] flat slots holding cached tokens
    cached_k: np.ndarray             # uint16 [n_cached, Hkv, D]
    cached_v: np.ndarray             # uint16 [n_cached, Hkv, D]
    poison: int                      # bf16 bit pattern of every other slot
    block_tables: np.ndarray         # int32  [num_seqs, max_blocks_per_seq], -1 = unused
    seq_lens: np.ndarray             # int32  [num_seqs]
    query_start_loc: np.ndarray      # int32  [num_seqs + 1]
    meta: dict = field(default_factory=dict)
    _pools: tuple = field(default=None, repr=False)

    # -- pools ---------------------------------------------------------------
    def _materialise(self):
        shape = (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)
        pools = []
        for rows in (self.cached_k, self.cached_v):
            pool = np.empty(shape, dtype=np.uint16)
            flat = pool.reshape(-1)
            n = flat.size
            bounds = [(i * n // _POOL_THREADS, (i + 1) * n // _POOL_THREADS) for i in range(_POOL_THREADS)]
            _par_map(lambda ab: flat[ab[0]:ab[1]].fill(self.poison), bounds)
            view = pool.reshape(-1, self.num_kv_heads, self.head_dim)
            view[self.cached_slots] = rows
            pools.append(pool)
        self._pools = tuple(pools)

    @property
    def k_cache(self) -> np.ndarray:
        """uint16 [NB, bs, Hkv, D]: the K pool before this step's kv_append."""
        if self._pools is None:
            self._materialise()
        return self._pools[0]

    @property
    def v_cache(self) -> np.ndarray:
        if self._pools is None:
            self._materialise()
        return self._pools[1]

    def drop_pools(self):
        self._pools = None

    # -- shapes --------------------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_q_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc).astype(np.int64)

    @property
    def max_query_len(self) -> int:
        ql = self.query_lens
        return int(ql.max()) if ql.size else 0

    def decode_seqs(self) -> np.ndarray:
        return np.nonzero(self.query_lens == 1)[0]

    def prefill_seqs(self) -> np.ndarray:
        return np.nonzero(self.query_lens > 1)[0]

    # -- accounting (bytes and pair counts of the workload; no attention math) --
    def kv_read_bytes(self, seqs=None) -> int:
        """K+V bytes an attention pass must read: every cached token once per sequence."""
        L = self.seq_lens.astype(np.int64)
        if seqs is not None:
            L = L[np.asarray(seqs, dtype=np.int64)]
        return int(L.sum()) * 2 * self.num_kv_heads * self.head_dim * 2

    def unique_kv_read_bytes(self, seqs=None) -> int:
        """Like kv_read_bytes but counting each physical block a shared prefix maps once."""
        idx = range(self.num_seqs) if seqs is None else [int(s) for s in seqs]
        seen = set()
        tokens = 0
        bs = self.block_size
        for s in idx:
            L = int(self.seq_lens[s])
            nb = (L + bs - 1) // bs
            for b in range(nb):
                phys = int(self.block_tables[s, b])
                n_tok = min(bs, L - b * bs)
                if phys in seen:
                    continue
                seen.add(phys)
                tokens += n_tok
        return tokens * 2 * self.num_kv_heads * self.head_dim * 2

    def causal_pairs(self, seqs=None) -> int:
        """Number of (query row, key) pairs with key position <= query position."""
        ql = self.query_lens
        L = self.seq_lens.astype(np.int64)
        idx = range(self.num_seqs) if seqs is None else seqs
        total = 0
        for s in idx:
            q = int(ql[s]); prior = int(L[s]) - q
            # rows j = 0..q-1 see prior + j + 1 keys
            total += q * (prior + 1) + q * (q - 1) // 2
        return total


def _rng(seed: int, cfg: int, stream: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg, stream, *extra])))


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


def _assemble(name, cfg_id, seed, Hq, Hkv, D, bs, seq_specs, num_blocks=None,
              share=None, row_order=None, outlier_frac=0.0, outlier_mult=8.0,
              placement_seed=None, poison=BF16_QNAN, extra_meta=None) -> Workload:
    """Build a workload from per-sequence (L, q) pairs.

    seq_specs: list of (seq_len_after_append, num_new_tokens), indexed by the
               original sequence id.
    share: None, (set_of_original_seq_ids, prefix_tokens), or a list of such
           groups, optionally (ids, prefix_tokens, {id: tokens}): the sequences
           of a group map one common set of blocks holding one common logical
           prefix of prefix_tokens tokens -- each its first `tokens` of them
           (all by default, a whole number of blocks), so that a member can leave
           the common prefix early and continue with blocks of its own.
    row_order: permutation of original sequence ids giving the batch order.
    """
    n = len(seq_specs)
    L0 = np.array([s[0] for s in seq_specs], dtype=np.int64)
    q0 = np.array([s[1] for s in seq_specs], dtype=np.int64)
    assert (q0 >= 0).all() and (q0 <= L0).all()
    nblk0 = (L0 + bs - 1) // bs

    if share is None:
        groups = []
    elif isinstance(share, list):
        groups = share
    else:
        groups = [share]
    share_of = {}                 # original id -> (group index, shared tokens)
    group_blocks = []             # blocks of each group's common prefix
    group_tokens = []
    for gi, grp in enumerate(groups):
        ids, prefix_tokens = grp[0], int(grp[1])
        own_tokens = grp[2] if len(grp) > 2 else {}
        assert prefix_tokens % bs == 0
        for s in ids:
            s = int(s)
            assert s not in share_of, "a sequence belongs to one sharing group"
            t = int(own_tokens.get(s, prefix_tokens))
            assert t % bs == 0 and 0 < t <= prefix_tokens
            assert L0[s] - q0[s] >= t, "new tokens must land past the shared prefix"
            share_of[s] = (gi, t)
        group_blocks.append(prefix_tokens // bs if ids else 0)
        group_tokens.append(prefix_tokens)
    sharers = set(share_of)
    share_blocks = group_blocks[0] if groups else 0
    unique_blocks = int(nblk0.sum()) - sum(t // bs for _, t in share_of.values()) + sum(
        b for gi, b in enumerate(group_blocks) if any(g == gi for g, _ in share_of.values()))
    if num_blocks is None:
        num_blocks = int(math.ceil(1.1 * unique_blocks))
    assert num_blocks >= unique_blocks

    # Block placement: one seeded permutation of the pool; sequences (in
    # original-id order) take consecutive disjoint slices, after the shared
    # prefix blocks of every group, which come first.
    prng = _rng(seed if placement_seed is None else placement_seed, cfg_id, _S_PLACEMENT)
    perm = prng.permutation(num_blocks).astype(np.int64)
    cursor = 0
    shared_ids_of = []
    for gi, b in enumerate(group_blocks):
        used = any(g == gi for g, _ in share_of.values())
        shared_ids_of.append(perm[cursor:cursor + b] if used else perm[:0])
        cursor += b if used else 0
    max_blocks = int(nblk0.max())
    bt0 = np.full((n, max_blocks), -1, dtype=np.int32)
    for s in range(n):
        if s in share_of:
            gi, t = share_of[s]
            sb = t // bs
            own = int(nblk0[s]) - sb
            bt0[s, :sb] = shared_ids_of[gi][:sb]
            bt0[s, sb:sb + own] = perm[cursor:cursor + own]
            cursor += own
        else:
            bt0[s, :nblk0[s]] = perm[cursor:cursor + nblk0[s]]
            cursor += int(nblk0[s])

    order = np.arange(n) if row_order is None else np.asarray(row_order, dtype=np.int64)
    assert sorted(order.tolist()) == list(range(n))

    # Batch index i holds original sequence order[i].
    L = L0[order]; qn = q0[order]; bt = bt0[order]
    qsl = np.zeros(n + 1, dtype=np.int64)
    qsl[1:] = np.cumsum(qn)
    T = int(qsl[-1])

    # the common prefix of each group that has members: its logical K/V and its cached slots
    prefix_kv = []
    shared_slots, shared_k, shared_v = [], [], []
    for gi, ptok in enumerate(group_tokens):
        if not any(g == gi for g, _ in share_of.values()):
            prefix_kv.append(None)
            continue
        r = _rng(seed, cfg_id, _S_KV, 1_000_000 + gi)
        pk = _normal_bf16(r, (ptok, Hkv, D))
        pv = _normal_bf16(r, (ptok, Hkv, D))
        prefix_kv.append((pk, pv))
        # slots of the prefix tokens some member maps
        used_tokens = max(t for g, t in share_of.values() if g == gi)
        pos = np.arange(used_tokens, dtype=np.int64)
        shared_slots.append(shared_ids_of[gi][pos // bs] * bs + pos % bs)
        shared_k.append(pk[:used_tokens])
        shared_v.append(pv[:used_tokens])
    if sharers and outlier_frac:
        raise NotImplementedError("outliers with a shared prefix are not generated")

    # Output buffers are allocated once and filled in place by the workers.
    prior_counts = np.array([int(L[i]) - int(qn[i]) - share_of.get(int(order[i]), (0, 0))[1]
                             for i in range(n)], dtype=np.int64)
    n_shared = int(sum(x.size for x in shared_slots))
    coff = np.zeros(n + 1, dtype=np.int64)
    coff[0] = n_shared
    coff[1:] = n_shared + np.cumsum(prior_counts)
    n_cached = int(coff[-1])
    q = np.empty((T, Hq, D), dtype=np.uint16)
    k_new = np.empty((T, Hkv, D), dtype=np.uint16)
    v_new = np.empty((T, Hkv, D), dtype=np.uint16)
    slots = np.empty(T, dtype=np.int64)
    cached_slots = np.empty(n_cached, dtype=np.int64)
    cached_k = np.empty((n_cached, Hkv, D), dtype=np.uint16)
    cached_v = np.empty((n_cached, Hkv, D), dtype=np.uint16)
    if n_shared:
        cached_slots[:n_shared] = np.concatenate(shared_slots)
        cached_k[:n_shared] = np.concatenate(shared_k)
        cached_v[:n_shared] = np.concatenate(shared_v)

    def one(i):
        s_orig = int(order[i])
        Ls, qs = int(L[i]), int(qn[i])
        prior = Ls - qs
        # Logical K/V for positions 0..Ls-1, keyed by the original sequence id
        # so that placement, block size and row order leave the data unchanged
        # (positions before `start` are the group's common prefix).
        r = _rng(seed, cfg_id, _S_KV, s_orig)
        start = share_of.get(s_orig, (0, 0))[1]
        kl = _normal_bf16(r, (Ls - start, Hkv, D))
        vl = _normal_bf16(r, (Ls - start, Hkv, D))
        if outlier_frac:
            ro = _rng(seed, cfg_id, _S_OUTLIER, s_orig)
            cnt = int(math.floor(outlier_frac * Ls))
            mult = np.float32(outlier_mult)
            for h in range(Hkv):
                pos = ro.choice(Ls, size=cnt, replace=False)
                # a power-of-two multiple of a bf16 value is exact in bf16
                vals = (kl[pos, h, :].astype(np.uint32) << np.uint32(16)).view(np.float32) * mult
                kl[pos, h, :] = f32_to_bf16_bits(vals)
        # kl/vl hold positions start..Ls-1; cached ones are start..prior-1
        a, b = int(coff[i]), int(coff[i + 1])
        pos = np.arange(start, prior, dtype=np.int64)
        cached_slots[a:b] = bt[i, pos // bs].astype(np.int64) * bs + pos % bs
        cached_k[a:b] = kl[:prior - start]
        cached_v[a:b] = vl[:prior - start]
        a, b = int(qsl[i]), int(qsl[i + 1])
        newpos = np.arange(prior, Ls, dtype=np.int64)
        slots[a:b] = bt[i, newpos // bs].astype(np.int64) * bs + newpos % bs
        k_new[a:b] = kl[prior - start:]
        v_new[a:b] = vl[prior - start:]
        rq = _rng(seed, cfg_id, _S_Q, s_orig)
        q[a:b] = _normal_bf16(rq, (qs, Hq, D))

    _par_map(one, range(n))

    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    pos_of = {int(s): int(i) for i, s in enumerate(order)}
    sharers_new = sorted(pos_of[s] for s in sharers)
    share_groups = [sorted(pos_of[s] for s, (g, _) in share_of.items() if g == gi) for gi in range(len(groups))]
    meta = dict(config=cfg_id, seed=seed, unique_blocks=unique_blocks,
                sharers=sharers_new, share_blocks=share_blocks, share_groups=share_groups)
    if extra_meta:
        meta.update(extra_meta)
    return Workload(name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                    num_blocks=num_blocks, scale=scale, q=q, k_new=k_new, v_new=v_new,
                    slot_mapping=slots, cached_slots=cached_slots, cached_k=cached_k,
                    cached_v=cached_v, poison=int(poison), block_tables=bt,
                    seq_lens=L.astype(np.int32), query_start_loc=qsl.astype(np.int32), meta=meta)


# ---------------------------------------------------------------------------
# The five task configurations
# ---------------------------------------------------------------------------

def config0(seed: int = 0, variant: str = "A", block_size: int = 16, placement_seed=None,
            poison=BF16_QNAN) -> Workload:
    """Tiny mixed batch: 4 sequences with contexts {1, 7, 16, 33}, Hq 4, Hkv 2, d 64.

    Reading A (default, 0-based "sequence 3"): sequences 0..2 take one decode
    row each (context 1, 7, 16 after the append); sequence 3 has 33 cached
    tokens and takes a 5-token causal chunk instead (38 after the append).
    Variant B (1-based): the chunk goes to the 16-token sequence (21 after).
    A sequence does not decode and prefill in the same step.
    """
    if variant == "A":
        specs = [(1, 1), (7, 1), (16, 1), (33 + 5, 5)]
    elif variant == "B":
        specs = [(1, 1), (7, 1), (16 + 5, 5), (33, 1)]
    else:
        raise ValueError(variant)
    return _assemble(f"tiny-{variant}", 0, seed, 4, 2, 64, block_size, specs, num_blocks=64,
                     placement_seed=placement_seed, poison=poison,
                     extra_meta=dict(variant=variant))


def config1(seed: int = 1, num_seqs: int = 64, placement_seed=None, block_size: int = 16,
            poison=BF16_QNAN) -> Workload:
    """Llama-3-8B-shaped decode layer: 64 seqs, context ~ U{128..4096}, Hq 32, Hkv 8, d 128.

    Pool = sum of blocks + 10%.  One decode row per sequence; kv_append of 64 tokens.
    """
    r = _rng(seed, 1, _S_LENGTHS)
    L = r.integers(128, 4096, size=num_seqs, endpoint=True)
    specs = [(int(x), 1) for x in L]
    return _assemble("llama3-8b-decode", 1, seed, 32, 8, 128, block_size, specs,
                     placement_seed=placement_seed, poison=poison)


def config2(seed: int = 2, num_seqs: int = 256, sigma: float = 1.0, placement_seed=None,
            poison=BF16_QNAN) -> Workload:
    """70B-class decode layer: 256 seqs, context lognormal(median 1024, sigma 1) capped at 8192.

    Hq 64, Hkv 8, d 128.  Per-layer KV bytes/token = 327,680 / 80 = 4,096; the
    pool holds the batch's blocks + 10% (the 95%-of-VRAM token budget of a
    whole 80-layer model cannot be the pool of a single layer).
    """
    r = _rng(seed, 2, _S_LENGTHS)
    raw = r.lognormal(mean=math.log(1024.0), sigma=sigma, size=num_seqs)
    L = np.clip(np.rint(raw), 1, 8192).astype(np.int64)
    specs = [(int(x), 1) for x in L]
    return _assemble("70b-decode", 2, seed, 64, 8, 128, 16, specs,
                     placement_seed=placement_seed, poison=poison,
                     extra_meta=dict(sigma=sigma))


def config3(seed: int = 3, num_prefill: int = 8, chunk: int = 512, num_decode: int = 192,
            prefix_tokens: int = 1024, num_sharers: int = 100, placement_seed=None,
            poison=BF16_QNAN) -> Workload:
    """Mixed continuous batch with a shared prefix, Llama-3-8B heads (32/8, d 128).

    8 chunked-prefill segments of 512 new tokens over cached prefixes P ~ U{0..2048}
    plus 192 decode rows with context ~ U{256..4096}.  Half of the 200 sequences
    (100, seeded choice among those whose cached part covers the 1024-token
    prefix) share the first 64 physical blocks.  Batch order is a seeded shuffle.
    """
    r = _rng(seed, 3, _S_LENGTHS)
    P = r.integers(0, 2048, size=num_prefill, endpoint=True)
    Ld = r.integers(256, 4096, size=num_decode, endpoint=True)
    specs = [(int(p) + chunk, chunk) for p in P] + [(int(x), 1) for x in Ld]
    n = len(specs)
    eligible = [s for s, (Ls, qs) in enumerate(specs) if Ls - qs >= prefix_tokens]
    rs = _rng(seed, 3, _S_SHARE)
    k = min(num_sharers, len(eligible))
    sharers = set(int(x) for x in rs.choice(np.array(eligible), size=k, replace=False)) if k else set()
    ro = _rng(seed, 3, _S_ORDER)
    order = ro.permutation(n)
    return _assemble("mixed-prefix", 3, seed, 32, 8, 128, 16, specs,
                     share=(sharers, prefix_tokens) if sharers else None, row_order=order,
                     placement_seed=placement_seed, poison=poison,
                     extra_meta=dict(eligible=len(eligible)))


def config4(seed: int = 4, num_seqs: int = 4, ctx: int = 131072, outlier_frac: float = 0.01,
            placement_seed=None, poison=BF16_QNAN) -> Workload:
    """Long-context decode: 4 seqs x 131072 tokens, Hq 64, Hkv 8, d 128.

    1% of keys scaled x8: for every (sequence, kv head), floor(0.01 * L) distinct
    positions (seeded) have their whole K row multiplied by 8 (exact in bf16).
    """
    specs = [(ctx, 1)] * num_seqs
    return _assemble("long-context-decode", 4, seed, 64, 8, 128, 16, specs,
                     outlier_frac=outlier_frac, placement_seed=placement_seed, poison=poison)


CONFIGS = {0: config0, 1: config1, 2: config2, 3: config3, 4: config4}


def make_config(i: int, **kw) -> Workload:
    return CONFIGS[i](**kw)


def custom(name: str, seq_specs, Hq: int, Hkv: int, D: int, bs: int, seed: int = 0,
           num_blocks=None, row_order=None, share=None, placement_seed=None,
           poison=BF16_QNAN, cfg_id: int = 99) -> Workload:
    """A workload from explicit (seq_len_after_append, new_tokens) pairs (tests, edge cases)."""
    return _assemble(name, cfg_id, seed, Hq, Hkv, D, bs, seq_specs, num_blocks=num_blocks,
                     row_order=row_order, share=share, placement_seed=placement_seed,
                     poison=poison)


# ---------------------------------------------------------------------------
# FP8 (E4M3) pools for the 8-bit cache
# ---------------------------------------------------------------------------

FP8_NAN = 0x7F     # E4M3 "FN" encoding: S.1111.111 is NaN, there are no infinities


@dataclass
class Fp8Pools:
    """K and V pools of 8-bit codes [NB, bs, Hkv, D] (uint8) with their per-pool scales.
    The already-cached rows hold random codes; every other slot holds ``poison``."""
    k_cache: np.ndarray
    v_cache: np.ndarray
    k_scale: float
    v_scale: float


def _fp8_code_draws(rng_of_chunk, n: int, center: int) -> np.ndarray:
    """n random E4M3 codes: random sign and mantissa, exponent field spread below
    ``center`` (a rounded normal with mean center - 1 and sd 1, clipped to
    1..center + 1, so magnitudes stay under 4 times 2^(center - 7) the way N(0,1)
    draws stay under a few units), about 1% with exponent field 0 (zeros and
    subnormals); never the NaN pattern.  Pure bit drawing: nothing is converted to or
    from a number.  Chunks of 2^22 codes are drawn in parallel, chunk i from the
    generator ``rng_of_chunk(i)``."""
    grid = np.arange(256) + 0.5
    top = min(15, center + 1)
    # exponent field of each 8-bit draw: inverse of a normal CDF sampled on 256 cells
    from math import erf, sqrt
    cdf = np.array([0.5 * (1 + erf((e + 0.5 - (center - 1)) / sqrt(2))) for e in range(1, top + 1)])
    e_of = np.searchsorted(cdf / cdf[-1], grid / 256.0, side="left") + 1
    e_of = np.minimum(e_of, top).astype(np.uint8)
    out = np.empty(n, dtype=np.uint8)
    step = 1 << 22

    def chunk(i):
        a = i * step
        b = min(n, a + step)
        r = rng_of_chunk(i).integers(0, 1 << 32, size=b - a, dtype=np.uint32)
        sign = ((r >> 7) & 1).astype(np.uint8)
        m = (r & 7).astype(np.uint8)
        e = e_of[(r >> 8) & 0xFF]
        e = np.where(((r >> 16) & 0xFF) < 3, np.uint8(0), e)
        m = np.where(e == 15, np.minimum(m, 6), m)            # keep clear of S.1111.111
        out[a:b] = (sign << 7) | (e << 3) | m

    _par_map(chunk, range((n + step - 1) // step))
    return out


def fp8_pools(wl: Workload, k_scale: float = 2.0 ** -4, v_scale: float = 2.0 ** -3,
              poison: int = FP8_NAN, seed: int = 0) -> Fp8Pools:
    """8-bit pools with the same block tables, lengths and cached slots as ``wl``.
    The exponent fields are centred so that code value x scale is of order 1."""
    shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim)
    cfg = int(wl.meta.get("config", 99))
    pools = []
    for which, sc in ((0, k_scale), (1, v_scale)):
        center = 7 + int(round(-math.log2(sc)))
        pool = np.full(shape, poison, dtype=np.uint8)
        rows = _fp8_code_draws(lambda i, which=which: _rng(seed, cfg, _S_FP8, which, i),
                               wl.cached_slots.size * wl.num_kv_heads * wl.head_dim, center)
        pool.reshape(-1, wl.num_kv_heads, wl.head_dim)[wl.cached_slots] = rows.reshape(
            -1, wl.num_kv_heads, wl.head_dim)
        pools.append(pool)
    return Fp8Pools(k_cache=pools[0], v_cache=pools[1], k_scale=float(np.float32(k_scale)),
                    v_scale=float(np.float32(v_scale)))
