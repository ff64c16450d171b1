"""GPU parity of paged_attention_append, the fused kv_append + paged_attention call.

Its contract is the two calls' result, bit for bit: on the same seeded inputs
the fused call must leave the pools and the output exactly as kv_append
followed by paged_attention does (over the whole pool), and the output is
also checked against the float64 oracle under the usual tolerance.  Row i of
k_new / v_new is the new token of query row i (the workloads' ordering).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_harness import DeviceBatch, compare, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import paged_kv_cache_tables_amd as pkv
    pkv.load_library()
    return torch


def fused(db, workspace=None):
    import paged_kv_cache_tables_amd as pkv
    pkv.paged_attention_append(db.out, db.q, db.k_new, db.v_new, db.slots, db.k_cache, db.v_cache, db.bt,
                               db.seq_lens, db.qsl, db.wl.scale, db.wl.max_query_len, workspace=workspace)


def check_fused_equals_separate(wl, label, oracle_rows="all"):
    import torch
    print(f"fused vs separate: {label}", flush=True)
    sep, fus = DeviceBatch(wl), DeviceBatch(wl)
    sep.step()                                    # kv_append, then paged_attention
    fused(fus)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(fus.k_cache), to_host_bits(sep.k_cache)), "K pool differs"
    assert np.array_equal(to_host_bits(fus.v_cache), to_host_bits(sep.v_cache)), "V pool differs"
    out = to_host_bits(fus.out)
    assert np.array_equal(out, to_host_bits(sep.out)), "output differs from the two separate calls"
    if oracle_rows is not None:
        rows = None if oracle_rows == "all" else oracle_rows
        k2, v2 = oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new, wl.slot_mapping)
        ref = oracle.paged_attention(wl.q, k2, v2, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                                     wl.num_kv_heads, wl.scale, rows=rows)
        compare(out, ref, rows=rows, label=f"fused-{label}")


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_fused_equals_separate_calls(cfg):
    check_fused_equals_separate(W.make_config(cfg), f"config{cfg}")


FUSED_EDGE = [
    ("bs8-mixed", [(1, 1), (9, 1), (700, 1), (130, 3), (300, 300)], 8, 2, 128, 8),
    ("bs32-g8", [(33, 1), (1025, 1), (2000, 64), (64, 64)], 16, 2, 128, 32),
    ("d64-mha", [(5, 1), (513, 1), (100, 37), (1, 1)], 4, 4, 64, 16),
    ("multi-row-g4", [(700, 4), (5, 2), (1300, 3), (64, 4), (2, 2), (900, 1)], 16, 4, 128, 16),
    ("block-boundary", [(16, 1), (17, 1), (64, 1), (65, 1), (32, 2), (80, 16)], 8, 8, 128, 16),
    ("long-many-pieces", [(100000, 1), (3, 1)], 8, 2, 128, 16),
    # a chunk over a long prefix: its items cut into pieces (partials in the decode rows'
    # workspace, after the merge launch has consumed them), decode rows beside it
    ("split-prefill", [(20000 + 64, 64), (3000, 1), (700, 1)], 32, 8, 128, 16),
]


@pytest.mark.parametrize("name,specs,Hq,Hkv,D,bs", FUSED_EDGE, ids=[e[0] for e in FUSED_EDGE])
def test_fused_edge_shapes(name, specs, Hq, Hkv, D, bs):
    check_fused_equals_separate(W.custom(name, specs, Hq, Hkv, D, bs, seed=len(name) + 7), name)


def test_fused_rows_out_of_order_and_empty_sequences():
    specs = [(40, 1), (25, 0), (300, 20), (9, 0), (1, 1), (200, 1)]
    wl = W.custom("fused-zero-rows", specs, 8, 2, 128, 16, seed=5, row_order=[3, 0, 5, 2, 1, 4])
    check_fused_equals_separate(wl, "zero-rows")


def test_fused_step_captured_in_hip_graph(gpu):
    """The fused step captured once and replayed: each replay (fresh pools and queries written
    by eager work in between) equals the eager fused call bit for bit."""
    torch = gpu
    import paged_kv_cache_tables_amd as pkv
    wl = W.config1(num_seqs=16)
    db = DeviceBatch(wl)
    k0, v0 = db.k_cache.clone(), db.v_cache.clone()
    need = pkv.workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                               wl.max_blocks_per_seq, wl.block_size, wl.max_query_len)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    q_alt = [db.q.clone(), torch.flip(db.q, dims=[1]).contiguous()]

    def reset(qv):
        db.k_cache.copy_(k0)
        db.v_cache.copy_(v0)
        db.q.copy_(qv)
        db.out.zero_()

    want = []
    for qv in q_alt:
        reset(qv)
        fused(db, ws)
        torch.cuda.synchronize()
        want.append((to_host_bits(db.out), to_host_bits(db.k_cache)))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fused(db, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fused(db, ws)
    torch.cuda.synchronize()
    for rep in range(4):
        i = rep % len(q_alt)
        reset(q_alt[i])
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(db.out), want[i][0]), f"replay {rep} output differs"
        assert np.array_equal(to_host_bits(db.k_cache), want[i][1]), f"replay {rep} pool differs"


def random_batch(seed):
    """A seeded batch whose shape the fixed cases do not cover: KV-head counts that are not powers
    of two (the decode workgroups then take 1 or 2 or 4 heads together), a random mix of rows per
    sequence (none, one, a few, a long chunk) and, half of the time, a shared prefix."""
    rng = np.random.default_rng(1000 + seed)
    Hkv = int(rng.choice([1, 2, 3, 4, 6, 8, 12]))
    G = int(rng.choice([g for g in (1, 2, 4, 8, 16) if Hkv * g <= 64]))
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([8, 16, 32]))
    n = int(rng.integers(1, 40))
    specs = []
    for _ in range(n):
        kind = rng.random()
        if kind < 0.1:
            L, q = int(rng.integers(1, 300)), 0
        elif kind < 0.6:
            L, q = int(rng.integers(1, 3000)), 1
        elif kind < 0.8:
            q = int(rng.integers(2, 9))
            L = q + int(rng.integers(0, 2000))
        else:
            q = int(rng.integers(9, 300))
            L = q + int(rng.integers(0, 1500))
        specs.append((L, q))
    share = None
    if rng.random() < 0.5:
        prefix = bs * int(rng.integers(1, 8))
        sharers = [i for i, (L, q) in enumerate(specs) if L - q >= prefix]
        if len(sharers) >= 2:
            share = (set(sharers), prefix)
    order = rng.permutation(n).tolist()
    name = f"random-{seed}-hkv{Hkv}-g{G}-d{D}-bs{bs}-n{n}"
    return W.custom(name, specs, Hkv * G, Hkv, D, bs, seed=seed, row_order=order, share=share)


@pytest.mark.parametrize("seed", range(12))
def test_fused_and_separate_on_random_batches(seed):
    wl = random_batch(seed)
    if wl.num_q_tokens == 0:
        pytest.skip("batch without rows")
    check_fused_equals_separate(wl, wl.name)
