"""Pins for the CPU oracle: each checks it against something other than itself.

* printed byte counts from the pages (tests/golden/kv_bytes_per_token.json);
* brute-force scalar attention (pure Python floats, no NumPy) on tiny inputs
  built from unpaged logical K/V;
* torch's scaled_dot_product_attention in float64 on CPU with KV heads
  repeated and an explicit boolean causal mask (a library routine);
* closed forms: length-1 context returns V exactly, a zero query averages V,
  identical keys average V;
* invariants: physical placement and block size, GQA = repeated-KV MHA,
  chunk splitting, decode row = last prefill row, shared prefix = private
  copy, poisoned tails and free blocks do not matter;
* append: bit copy round trip, untouched slots, padding slots, errors.

``test_planted_mistakes_are_caught`` plants typical mistakes in the oracle's
steps (on the CPU) and checks that the pins catch every one.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import paged as O
import workloads as W

ORACLE_PINS = []


def pin(fn):
    ORACLE_PINS.append(fn)
    return fn


# ---------------------------------------------------------------------------
# helpers: build paged inputs from logical per-sequence K/V (test-side code)
# ---------------------------------------------------------------------------

def _bits(x):
    return W.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _f(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def make_paged(seqs, Hq, Hkv, D, bs, seed=0, place_seed=None, num_blocks=None, poison=W.BF16_QNAN,
               logical=None):
    """seqs: list of (L, q_len).  Returns dict with logical f64 K/V, bits, pools, tables."""
    rng = np.random.default_rng(seed)
    if logical is None:
        logical = []
        for (L, ql) in seqs:
            k = _bits(rng.standard_normal((L, Hkv, D)))
            v = _bits(rng.standard_normal((L, Hkv, D)))
            logical.append((k, v))
    nblk = [(L + bs - 1) // bs for (L, _) in seqs]
    need = sum(nblk)
    NB = num_blocks or need + 3
    prng = np.random.default_rng(1000 + (seed if place_seed is None else place_seed))
    perm = prng.permutation(NB)
    kp = np.full((NB, bs, Hkv, D), poison, np.uint16)
    vp = np.full((NB, bs, Hkv, D), poison, np.uint16)
    bt = np.full((len(seqs), max(nblk)), -1, np.int32)
    c = 0
    for s, (L, ql) in enumerate(seqs):
        ids = perm[c:c + nblk[s]]; c += nblk[s]
        bt[s, :nblk[s]] = ids
        k, v = logical[s]
        for t in range(L):
            kp[ids[t // bs], t % bs] = k[t]
            vp[ids[t // bs], t % bs] = v[t]
    qsl = np.zeros(len(seqs) + 1, np.int64)
    qsl[1:] = np.cumsum([ql for (_, ql) in seqs])
    q = _bits(rng.standard_normal((int(qsl[-1]), Hq, D)))
    return dict(q=q, kp=kp, vp=vp, bt=bt, L=np.array([L for L, _ in seqs], np.int32),
                qsl=qsl.astype(np.int32), logical=logical, Hq=Hq, Hkv=Hkv, D=D, bs=bs)


def run_oracle(P, scale, **kw):
    return oracle.paged_attention(P["q"], P["kp"], P["vp"], P["bt"], P["L"], P["qsl"], P["Hkv"], scale, **kw)


def brute_force(P, scale):
    """Scalar Python attention from the logical (unpaged) data."""
    Hq, Hkv, D = P["Hq"], P["Hkv"], P["D"]
    G = Hq // Hkv
    out = {}
    qf = _f(P["q"])
    for s, (k, v) in enumerate(P["logical"]):
        kf, vf = _f(k), _f(v)
        a, b = int(P["qsl"][s]), int(P["qsl"][s + 1])
        L = int(P["L"][s])
        for j in range(b - a):
            pos = L - (b - a) + j
            for g in range(Hq):
                h = g // G
                z = []
                for t in range(pos + 1):
                    acc = 0.0
                    for d in range(D):
                        acc += float(qf[a + j, g, d]) * float(kf[t, h, d])
                    z.append(float(np.float32(scale)) * acc)
                m = max(z)
                e = [math.exp(x - m) for x in z]
                tot = sum(e)
                out[(a + j, g)] = [sum(e[t] * float(vf[t, h, d]) for t in range(pos + 1)) / tot
                                   for d in range(D)]
    return out


TINY = [(1, 1), (5, 1), (9, 3), (13, 13), (20, 4)]


# ---------------------------------------------------------------------------
# O1: bytes per token
# ---------------------------------------------------------------------------

def test_kv_bytes_per_token_matches_printed_values(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "kv_bytes_per_token.json")))
    for case in g["per_token"]:
        assert oracle.kv_bytes_per_token(*case["args"]) == case["expected"], case["cite"]
    for case in g["totals"]:
        got = oracle.kv_bytes_per_token(*case["args"]) * case["tokens"] / case["divisor"]
        assert got == case["expected"], case["cite"]
    for case in g["per_block"]:
        assert oracle.kv_bytes_per_token(*case["args"]) * case["block_size"] == case["expected"], case["cite"]


def test_kv_bytes_per_token_invalid_arguments():
    for bad in [(0, 8, 128, 2), (80, 0, 128, 2), (80, 8, -1, 2), (80, 8, 128, 0)]:
        assert oracle.kv_bytes_per_token(*bad) == -1


# ---------------------------------------------------------------------------
# O3 pins (each returns None or raises AssertionError, so the planted-mistake
# test can run them against a mutated oracle)
# ---------------------------------------------------------------------------

@pin
def pin_brute_force_tiny():
    for (Hq, Hkv, D, bs) in [(4, 2, 8, 4), (3, 1, 6, 8), (2, 2, 5, 2)]:
        P = make_paged(TINY, Hq, Hkv, D, bs, seed=Hq * 10 + D)
        scale = 1.0 / math.sqrt(D)
        got = run_oracle(P, scale)
        ref = brute_force(P, scale)
        for (r, g), vec in ref.items():
            np.testing.assert_allclose(got[r, g], vec, rtol=1e-12, atol=1e-12)


@pin
def pin_torch_sdpa_dense():
    import torch
    for (Hq, Hkv, D, bs) in [(8, 2, 16, 4), (4, 4, 32, 16)]:
        P = make_paged([(37, 37), (50, 9), (17, 1)], Hq, Hkv, D, bs, seed=7 + D)
        scale = float(np.float32(1.0 / math.sqrt(D)))
        got = run_oracle(P, scale)
        G = Hq // Hkv
        for s, (k, v) in enumerate(P["logical"]):
            a, b = int(P["qsl"][s]), int(P["qsl"][s + 1])
            L = int(P["L"][s]); ql = b - a
            qt = torch.from_numpy(_f(P["q"][a:b])).permute(1, 0, 2)[None]          # [1,Hq,ql,D]
            kt = torch.from_numpy(_f(k)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
            vt = torch.from_numpy(_f(v)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
            pos = torch.arange(L - ql, L)[:, None]
            mask = torch.arange(L)[None, :] <= pos                                   # [ql, L]
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
            np.testing.assert_allclose(got[a:b], ref[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


@pin
def pin_length_one_returns_v():
    P = make_paged([(1, 1), (1, 1)], 4, 2, 16, 16, seed=3)
    got = run_oracle(P, 0.25)
    for s, (k, v) in enumerate(P["logical"]):
        for g in range(4):
            assert np.array_equal(got[s, g], _f(v)[0, g // 2])


@pin
def pin_zero_query_averages_v():
    P = make_paged([(11, 3), (6, 1)], 4, 2, 8, 4, seed=5)
    P["q"][:] = 0
    got = run_oracle(P, 0.5)
    for s, (k, v) in enumerate(P["logical"]):
        a, b = int(P["qsl"][s]), int(P["qsl"][s + 1]); L = int(P["L"][s])
        for j in range(b - a):
            p = L - (b - a) + j
            for g in range(4):
                np.testing.assert_allclose(got[a + j, g], _f(v)[:p + 1, g // 2].mean(0), rtol=1e-13, atol=1e-14)


@pin
def pin_identical_keys_average_v():
    rng = np.random.default_rng(11)
    L = 9
    k = np.repeat(_bits(rng.standard_normal((1, 2, 8))), L, axis=0)
    v = _bits(rng.standard_normal((L, 2, 8)))
    P = make_paged([(L, 4)], 4, 2, 8, 4, seed=11, logical=[(k, v)])
    got = run_oracle(P, 0.3)
    for j in range(4):
        p = L - 4 + j
        for g in range(4):
            np.testing.assert_allclose(got[j, g], _f(v)[:p + 1, g // 2].mean(0), rtol=1e-13, atol=1e-14)


@pin
def pin_placement_and_block_size_invariance():
    base = make_paged(TINY, 4, 2, 8, 16, seed=21)
    ref = run_oracle(base, 0.35)
    for bs in (1, 4, 8, 16, 32):
        for ps in (0, 1, 2):
            P = make_paged(TINY, 4, 2, 8, bs, seed=21, place_seed=ps, logical=base["logical"],
                           num_blocks=sum((L + bs - 1) // bs for L, _ in TINY) + 7)
            P["q"] = base["q"]
            got = run_oracle(P, 0.35)
            assert np.array_equal(got, ref), (bs, ps)


@pin
def pin_gqa_equals_repeated_kv_mha():
    P = make_paged(TINY, 8, 2, 8, 4, seed=31)
    got = run_oracle(P, 0.3)
    rep = dict(P)
    rep["kp"] = np.repeat(P["kp"], 4, axis=2)
    rep["vp"] = np.repeat(P["vp"], 4, axis=2)
    rep["Hkv"] = 8
    # per-head vs per-group matrix products may sum in another order: equal to rounding
    np.testing.assert_allclose(run_oracle(rep, 0.3), got, rtol=1e-13, atol=1e-15)


@pin
def pin_chunk_split_and_decode_equals_last_prefill_row():
    # one 12-row chunk over an 8-token prefix vs two 6-row chunks vs 12 decode steps
    L = 20
    P = make_paged([(L, 12)], 4, 2, 8, 4, seed=41)
    full = run_oracle(P, 0.3)
    q = P["q"]
    for split in (6, 1):
        rows = []
        for start in range(0, 12, split):
            Q = dict(P)
            Q["q"] = q[start:start + split]
            Q["L"] = np.array([L - 12 + start + split], np.int32)
            Q["qsl"] = np.array([0, split], np.int32)
            rows.append(run_oracle(Q, 0.3))
        assert np.array_equal(np.concatenate(rows), full)


@pin
def pin_prefix_sharing_equals_private_copy():
    rng = np.random.default_rng(51)
    Hkv, D, bs = 2, 8, 4
    prefix_k = _bits(rng.standard_normal((8, Hkv, D)))
    prefix_v = _bits(rng.standard_normal((8, Hkv, D)))
    logical = []
    for L in (13, 10):
        k = np.concatenate([prefix_k, _bits(rng.standard_normal((L - 8, Hkv, D)))])
        v = np.concatenate([prefix_v, _bits(rng.standard_normal((L - 8, Hkv, D)))])
        logical.append((k, v))
    P = make_paged([(13, 2), (10, 1)], 4, Hkv, D, bs, seed=51, logical=logical, num_blocks=12)
    private = run_oracle(P, 0.3)
    # re-point sequence 1's first two table entries at sequence 0's prefix blocks
    S = dict(P)
    S["bt"] = P["bt"].copy()
    S["bt"][1, :2] = P["bt"][0, :2]
    S["kp"] = P["kp"].copy(); S["vp"] = P["vp"].copy()
    S["kp"][P["bt"][1, :2]] = W.BF16_QNAN   # the now-unreferenced private copy is garbage
    S["vp"][P["bt"][1, :2]] = W.BF16_QNAN
    assert np.array_equal(run_oracle(S, 0.3), private)


@pin
def pin_poisoned_tails_do_not_matter():
    ref = run_oracle(make_paged(TINY, 4, 2, 8, 8, seed=61, poison=np.uint16(0)), 0.3)
    for poison in (W.BF16_QNAN, W.BF16_PINF, W.BF16_NINF):
        got = run_oracle(make_paged(TINY, 4, 2, 8, 8, seed=61, poison=poison), 0.3)
        assert np.array_equal(got, ref)
        assert np.isfinite(got).all()


@pin
def pin_scale_enters_linearly_in_the_logits():
    # softmax(c * z) with c -> 0 averages V; large c approaches argmax selection
    P = make_paged([(7, 1)], 2, 1, 8, 4, seed=71)
    k, v = P["logical"][0]
    kf, vf, qf = _f(k), _f(v), _f(P["q"])
    got = run_oracle(P, 1e-30)
    np.testing.assert_allclose(got[0, 0], vf[:, 0].mean(0), rtol=1e-12)
    got = run_oracle(P, 1e4)
    best = int(np.argmax(kf[:, 0] @ qf[0, 0]))
    np.testing.assert_allclose(got[0, 0], vf[best, 0], rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("fn", ORACLE_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(fn):
    fn()


# ---------------------------------------------------------------------------
# Planted mistakes: every one must make at least one pin fail
# ---------------------------------------------------------------------------

def _mut_head_mod(g, group):
    return g % 2                        # interleaved instead of contiguous grouping


def _mut_pos_off_by_one(L, q, j):
    return L - q + j - 1                # drops the newest key


def _mut_pos_ignores_chunk(L, q, j):
    return L - 1                         # every chunk row sees the whole chunk (no causal mask)


def _mut_softmax_no_scale(qh, K, V, scale):
    z = qh @ K.T
    w = np.exp(z - z.max(axis=1, keepdims=True))
    return (w @ V) / w.sum(axis=1, keepdims=True)


def _mut_softmax_kt_swapped(qh, K, V, scale):
    z = scale * (qh @ V.T)               # keys and values swapped
    w = np.exp(z - z.max(axis=1, keepdims=True))
    return (w @ K) / w.sum(axis=1, keepdims=True)


def _mut_softmax_unnormalised(qh, K, V, scale):
    z = scale * (qh @ K.T)
    w = np.exp(z - z.max(axis=1, keepdims=True))
    return w @ V


def _mut_gather_logical(pool, table_row, n):
    bs = pool.shape[1]
    out = np.empty((n,) + pool.shape[2:], dtype=np.uint16)
    for b in range((n + bs - 1) // bs):
        cnt = min(bs, n - b * bs)
        out[b * bs:b * bs + cnt] = pool[b, :cnt]         # ignores the table
    return out


def _mut_gather_reversed_offsets(pool, table_row, n):
    bs = pool.shape[1]
    out = np.empty((n,) + pool.shape[2:], dtype=np.uint16)
    for t in range(n):
        out[t] = pool[int(table_row[t // bs]), bs - 1 - t % bs]   # wrong in-block offset
    return out


MUTANTS = [
    ("kv_head_of", _mut_head_mod),
    ("row_position", _mut_pos_off_by_one),
    ("row_position", _mut_pos_ignores_chunk),
    ("softmax_attend", _mut_softmax_no_scale),
    ("softmax_attend", _mut_softmax_kt_swapped),
    ("softmax_attend", _mut_softmax_unnormalised),
    ("gather_tokens", _mut_gather_logical),
    ("gather_tokens", _mut_gather_reversed_offsets),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_planted_mistakes_are_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(O, name, mutant)
    caught = []
    for fn in ORACLE_PINS:
        try:
            fn()
        except Exception:                 # assertion, shape error or NaN check
            caught.append(fn.__name__)
    assert caught, f"no pin catches the planted mistake {mutant.__name__}"


# ---------------------------------------------------------------------------
# Split-K identity (the method's rescale step, in float64): merging per-split
# partial (o, m, l) reproduces the oracle for any split size.
# ---------------------------------------------------------------------------

def test_split_merge_identity_float64():
    P = make_paged([(300, 1), (77, 1)], 8, 2, 16, 16, seed=81)
    scale = 0.25
    ref = run_oracle(P, scale)
    qf = _f(P["q"])
    for S in (1, 16, 64, 100, 512):
        for s, (k, v) in enumerate(P["logical"]):
            kf, vf = _f(k), _f(v)
            L = int(P["L"][s])
            for g in range(8):
                h = g // 4
                parts = []
                for t0 in range(0, L, S):
                    z = scale * (kf[t0:t0 + S, h] @ qf[s, g])
                    m = z.max()
                    e = np.exp(z - m)
                    parts.append((e @ vf[t0:t0 + S, h], m, e.sum()))
                M = max(p[1] for p in parts)
                num = sum(o * math.exp(m - M) for o, m, l in parts)
                den = sum(l * math.exp(m - M) for o, m, l in parts)
                np.testing.assert_allclose(num / den, ref[s, g], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# O2: append
# ---------------------------------------------------------------------------

def test_append_round_trip_and_untouched_slots():
    Wl = W.config0()
    k2, v2 = oracle.kv_append(Wl.k_cache, Wl.v_cache, Wl.k_new, Wl.v_new, Wl.slot_mapping,
                              Wl.block_tables, Wl.seq_lens)
    # round trip: walking the table at the new positions returns the new rows bitwise
    for s in range(Wl.num_seqs):
        a, b = int(Wl.query_start_loc[s]), int(Wl.query_start_loc[s + 1])
        L = int(Wl.seq_lens[s])
        rows = O.gather_tokens(k2, Wl.block_tables[s], L)[L - (b - a):]
        assert np.array_equal(rows, Wl.k_new[a:b])
        rows = O.gather_tokens(v2, Wl.block_tables[s], L)[L - (b - a):]
        assert np.array_equal(rows, Wl.v_new[a:b])
    # every other slot is unchanged
    touched = np.zeros(Wl.num_blocks * Wl.block_size, bool)
    touched[Wl.slot_mapping] = True
    flat_before = Wl.k_cache.reshape(-1, Wl.num_kv_heads, Wl.head_dim)
    flat_after = k2.reshape(-1, Wl.num_kv_heads, Wl.head_dim)
    assert np.array_equal(flat_before[~touched], flat_after[~touched])


def test_append_padding_and_errors():
    Wl = W.config0()
    slots = Wl.slot_mapping.copy()
    slots[2] = -1
    k2, _ = oracle.kv_append(Wl.k_cache, Wl.v_cache, Wl.k_new, Wl.v_new, slots)
    assert np.array_equal(k2.reshape(-1, 2, 64)[Wl.slot_mapping[2]],
                          Wl.k_cache.reshape(-1, 2, 64)[Wl.slot_mapping[2]])
    dup = Wl.slot_mapping.copy(); dup[1] = dup[0]
    with pytest.raises(ValueError):
        oracle.kv_append(Wl.k_cache, Wl.v_cache, Wl.k_new, Wl.v_new, dup)
    oob = Wl.slot_mapping.copy(); oob[0] = Wl.num_blocks * Wl.block_size
    with pytest.raises(ValueError):
        oracle.kv_append(Wl.k_cache, Wl.v_cache, Wl.k_new, Wl.v_new, oob)


def test_append_into_shared_block_is_an_error():
    bt = np.array([[3, 4], [3, 5]], np.int32)
    pool = np.zeros((8, 4, 1, 2), np.uint16)
    new = np.ones((1, 1, 2), np.uint16)
    with pytest.raises(ValueError):
        oracle.kv_append(pool, pool, new, new, np.array([3 * 4 + 1]), bt, np.array([6, 6]))


def test_query_rows_beyond_length_rejected():
    P = make_paged([(3, 3)], 2, 1, 4, 4)
    P["L"] = np.array([2], np.int32)
    with pytest.raises(ValueError):
        run_oracle(P, 0.5)
