"""GPU parity: the HIP library (through the C ABI) against the float64 CPU oracle.

Bars: kv_append is bit-exact over the whole pool; attention is within
1e-2 max abs per element (one bf16 ulp of the reference only where the
correctly rounded bf16 value is itself more than 1e-2 away, which needs
|ref| >= 4) and 1e-3 mean abs.  Every row of every configuration is checked
against the oracle.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_harness import DeviceBatch, bf16_to_f64, compare, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import paged_kv_cache_tables_amd as pkv
    pkv.load_library()
    return torch


def oracle_after_append(wl):
    return oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new, wl.slot_mapping)


def run_and_check(wl, rows=None, label=""):
    db = DeviceBatch(wl)
    db.step()
    import torch
    torch.cuda.synchronize()
    k2, v2 = oracle_after_append(wl)
    ref = oracle.paged_attention(wl.q, k2, v2, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                                 wl.num_kv_heads, wl.scale, rows=rows)
    out = to_host_bits(db.out)
    stats = compare(out, ref, rows=rows, label=label or wl.name)
    return db, out, stats


# ---------------------------------------------------------------------------
# kv_append: bit-exact over the whole pool
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_append_bit_exact_whole_pool(cfg):
    print(f"append config {cfg}", flush=True)
    wl = W.make_config(cfg)
    db = DeviceBatch(wl)
    db.append()
    k2, v2 = oracle_after_append(wl)
    assert np.array_equal(to_host_bits(db.k_cache), k2)
    assert np.array_equal(to_host_bits(db.v_cache), v2)


def test_append_skips_padding_slots():
    wl = W.config0()
    wl.slot_mapping = wl.slot_mapping.copy()
    wl.slot_mapping[[1, 4]] = -1
    db = DeviceBatch(wl)
    db.append()
    k2, v2 = oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new, wl.slot_mapping)
    assert np.array_equal(to_host_bits(db.k_cache), k2)
    assert np.array_equal(to_host_bits(db.v_cache), v2)


# ---------------------------------------------------------------------------
# attention parity on the five configurations
# ---------------------------------------------------------------------------

def test_config0_all_rows_and_length_one_exact():
    wl = W.config0()
    db, out, stats = run_and_check(wl)
    # sequence 0 has a single token: the output is its V row, bit for bit
    G = wl.num_q_heads // wl.num_kv_heads
    for g in range(wl.num_q_heads):
        assert np.array_equal(out[0, g], wl.v_new[0, g // G])


def test_config0_variant_b():
    run_and_check(W.config0(variant="B"))


def test_config1_llama8b_decode_all_rows():
    run_and_check(W.config1())


def test_config2_70b_decode_all_rows():
    run_and_check(W.config2())


def test_config3_mixed_prefix_all_rows():
    run_and_check(W.config3())


def test_config4_long_context_all_rows():
    wl = W.config4()
    run_and_check(wl)


def test_config4_single_sequence_512_token_pieces():
    """One 131072-token sequence with the long-context heads (64 query, 8 KV, d 128) and 1% of
    its keys scaled x8: the decode waves' equal shares are then exactly 512 keys, so every
    (sequence, head) is merged from 256 pieces of 512 keys, the configuration's stated split."""
    wl = W.config4(num_seqs=1)
    _, _, stats = run_and_check(wl, label="long-context-1x131072")
    assert stats["n"] == 64 * 128


# ---------------------------------------------------------------------------
# shapes and edge cases
# ---------------------------------------------------------------------------

EDGE = [
    # name, seq_specs (L, q), Hq, Hkv, D, bs
    ("bs8-d128-g4", [(1, 1), (9, 1), (700, 1), (130, 3), (300, 300)], 8, 2, 128, 8),
    ("bs32-d128-g8", [(33, 1), (1025, 1), (2000, 64), (64, 64)], 16, 2, 128, 32),
    ("d64-g1-mha", [(5, 1), (513, 1), (100, 37), (1, 1)], 4, 4, 64, 16),
    ("d64-g16", [(17, 1), (4000, 1), (200, 150)], 16, 1, 64, 16),
    ("d128-g2", [(2, 2), (3, 1), (65, 65), (1100, 1)], 4, 2, 128, 16),
    ("mqa-d128-g16", [(777, 1), (300, 130)], 16, 1, 128, 16),
    ("split-tails", [(511, 1), (512, 1), (513, 1), (1023, 1), (1024, 1), (1025, 1), (64, 1), (65, 1)],
     8, 2, 128, 16),
    ("long-single", [(20000, 1)], 32, 8, 128, 16),
    ("chunk-from-zero", [(512, 512), (97, 97)], 32, 8, 128, 16),
    # decode work is cut into equal shares of (sequence, KV head, 64-token tile) units:
    # many short sequences (a lane scans several, a share spans many segments) ...
    ("many-short-decode", [(1 + (i * 37) % 130, 1) for i in range(300)], 8, 2, 128, 16),
    # ... decode rows around prefill rows that the partition skips ...
    ("decode-around-prefill", [(41 + (i * 211) % 900, 1 if i % 7 else 40) for i in range(90)], 16, 4, 128, 16),
    # ... and long sequences cut into ~200 pieces (the merge's wide form), d 128 and d 64
    ("long-many-pieces", [(100000, 1)], 8, 2, 128, 16),
    ("long-d64-wide-merge", [(40000, 1), (3, 1)], 8, 2, 64, 16),
    # short chunks (q_s x G <= 16, e.g. speculative verification) run with the decode rows:
    # every row its own causal limit, pieces and merge per (sequence, row, head)
    ("multi-row-g4", [(700, 4), (5, 2), (1300, 3), (64, 4), (2, 2), (900, 1)], 16, 4, 128, 16),
    ("multi-row-g8", [(3000, 2), (17, 2), (600, 1)], 64, 8, 128, 16),
    ("multi-row-g2-d64", [(2500, 8), (9, 8), (300, 5)], 8, 4, 64, 16),
    ("multi-row-mha", [(1500, 16), (16, 16), (40, 7)], 4, 4, 128, 16),
    ("spec-verify-long", [(20000 + 997 * i, 4) for i in range(6)], 32, 8, 128, 16),
    ("short-and-long-chunks", [(800, 4), (1000, 300), (2000, 1), (90, 3), (513, 64)], 32, 8, 128, 16),
    # the planner lists up to 256 sequences with chunk rows and hands their items out one per
    # thread; exactly 256 of them among decode rows, and 300 (one thread per sequence)
    ("prefill-chunks-256", [(50 + (i * 41) % 300, 3 if i % 5 == 0 else 20) for i in range(320)],
     8, 2, 128, 16),
    ("prefill-chunks-300", [(30 + (i * 67) % 400, 17 + i % 16) for i in range(300)], 8, 2, 128, 16),
]


@pytest.mark.parametrize("name,specs,Hq,Hkv,D,bs", EDGE, ids=[e[0] for e in EDGE])
def test_edge_shapes(name, specs, Hq, Hkv, D, bs):
    wl = W.custom(name, specs, Hq, Hkv, D, bs, seed=len(name))
    run_and_check(wl)


# Chunks over long prefixes with few items for the device: the planner cuts each item of more
# than 64 key tiles into pieces of consecutive tiles (one workgroup each, partials merged by the
# last piece to finish).  Cases: pieces with d 128 / G 4, d 64 / G 1 (128-row items), G 16
# (8-row items), a split item among short chunk items and decode rows, a batch whose first
# split length would need more partial slots than the workspace holds (the length is doubled,
# every item still cut in two; rows sampled, the oracle being slow at that size), and KV head
# counts of 6 and 16 (partial slots per head 85 and 32), a split item among more chunks than
# the planner's sequence list holds, and block sizes 8 and 32.
SPLIT = [
    ("split-long-prefix", [(20000 + 64, 64), (3000, 1), (500, 1)], 32, 8, 128, 16, None),
    ("split-d64-mha", [(12000 + 128, 128), (700, 1)], 8, 8, 64, 16, None),
    ("split-g16", [(9000 + 40, 40)], 16, 1, 128, 16, None),
    ("split-among-short-items", [(40000 + 100, 100), (600, 300), (200, 200), (5000, 1), (70, 1)],
     32, 8, 128, 16, None),
    ("split-length-doubled", [(8600 + 128, 128)] * 30, 8, 8, 64, 16, 48),
    # KV head counts that do not divide the partial slots evenly, and 16 heads of G 1
    ("split-hkv6-g2", [(15000 + 48, 48), (900, 1)], 12, 6, 128, 16, None),
    ("split-hkv16-g1", [(30000 + 128, 128)], 16, 16, 64, 16, 40),
    ("split-among-260-chunks", [(9000 + 5, 5)] + [(40 + (i * 53) % 300, 5) for i in range(260)],
     16, 1, 128, 16, None),
    # pool blocks of 8 and 32 tokens (a piece starts on a 64-key tile, so on a block boundary)
    ("split-bs8", [(9000 + 64, 64), (300, 1)], 32, 8, 128, 8, None),
    ("split-bs32-d64", [(12000 + 100, 100), (77, 1)], 16, 4, 64, 32, None),
]


@pytest.mark.parametrize("name,specs,Hq,Hkv,D,bs,nrows", SPLIT, ids=[e[0] for e in SPLIT])
def test_prefill_split_items(name, specs, Hq, Hkv, D, bs, nrows):
    wl = W.custom(name, specs, Hq, Hkv, D, bs, seed=len(name) + 100)
    rows = None
    if nrows is not None:
        rows = np.unique(np.random.default_rng(5).integers(0, wl.num_q_tokens, size=nrows))
    print(f"{name}: {wl.num_q_tokens} rows, checking {len(rows) if rows is not None else 'all'}", flush=True)
    run_and_check(wl, rows=rows)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.75], ids=["negative", "zero", "large"])
def test_any_finite_softmax_scale(scale):
    """The softmax scale is any finite float: negative (the prefill kernel negates the
    query instead, so that both paths take the row max of the scaled scores), zero (uniform
    weights) and large (weights concentrated on a few keys, several rescales of the running
    max), over decode rows, multi-row decode rows and prefill rows, d 128 and d 64."""
    import dataclasses
    for D in (128, 64):
        wl = W.custom(f"scale-{scale}-d{D}", [(700, 1), (130, 3), (300, 300), (1500, 64), (9, 1), (2100, 1)],
                      16, 4, D, 16, seed=D)
        wl = dataclasses.replace(wl, scale=float(np.float32(scale)))
        print(f"scale {wl.scale} d {D}", flush=True)
        run_and_check(wl)


def test_sequences_without_rows_and_interleaved_order():
    specs = [(40, 1), (25, 0), (300, 20), (9, 0), (1, 1), (200, 1)]
    wl = W.custom("zero-rows", specs, 8, 2, 128, 16, seed=3, row_order=[3, 0, 5, 2, 1, 4])
    run_and_check(wl)


def test_empty_batch_is_a_no_op(gpu):
    torch = gpu
    import paged_kv_cache_tables_amd as pkv
    k = torch.zeros((4, 16, 2, 64), dtype=torch.bfloat16, device="cuda:0")
    q = torch.zeros((0, 4, 64), dtype=torch.bfloat16, device="cuda:0")
    out = torch.zeros_like(q)
    i32 = dict(dtype=torch.int32, device="cuda:0")
    pkv.paged_attention(out, q, k, k, torch.zeros((0, 1), **i32), torch.zeros(0, **i32),
                        torch.zeros(1, **i32), 0.125, 0)
    pkv.kv_append(torch.zeros((0, 2, 64), dtype=torch.bfloat16, device="cuda:0"),
                  torch.zeros((0, 2, 64), dtype=torch.bfloat16, device="cuda:0"),
                  torch.zeros(0, dtype=torch.int64, device="cuda:0"), k, k)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# invariants on the GPU path
# ---------------------------------------------------------------------------

def test_poisoned_slots_do_not_change_the_output():
    outs = []
    for poison in (W.BF16_QNAN, W.BF16_PINF, W.BF16_NINF, np.uint16(0)):
        wl = W.config0(poison=poison)
        db = DeviceBatch(wl)
        db.step()
        outs.append(to_host_bits(db.out))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    wl = W.custom("poison-mixed", [(70, 1), (300, 45), (1500, 1)], 8, 2, 128, 16, seed=9,
                  poison=W.BF16_PINF)
    wl2 = W.custom("poison-mixed", [(70, 1), (300, 45), (1500, 1)], 8, 2, 128, 16, seed=9,
                   poison=W.BF16_QNAN)
    a, b = DeviceBatch(wl), DeviceBatch(wl2)
    a.step(); b.step()
    assert np.array_equal(to_host_bits(a.out), to_host_bits(b.out))


def test_run_to_run_determinism():
    wl = W.config3()
    db = DeviceBatch(wl)
    db.step()
    first = to_host_bits(db.out)
    for _ in range(2):
        db.attend()
        assert np.array_equal(to_host_bits(db.out), first)


def test_prefix_sharing_equals_private_copies():
    """The mixed batch's 100 sharers map one 1024-token prefix; the decode rows among them are
    attended as sharing groups (the shared tiles read once per block of 16 query columns), so
    the shared layout and a copy of the prefix per sequence take different paths through the
    kernels: both must match the oracle, which gives both layouts the same float64 result."""
    wl = W.config3()
    db = DeviceBatch(wl)
    db.step()
    shared = to_host_bits(db.out)
    # give every sharer its own copy of the 64 prefix blocks
    sharers = wl.meta["sharers"]
    import torch
    extra = 64 * (len(sharers) - 1)
    NB2 = wl.num_blocks + extra
    k = torch.empty((NB2,) + db.k_cache.shape[1:], dtype=db.k_cache.dtype, device=db.k_cache.device)
    v = torch.empty_like(k)
    k[:wl.num_blocks] = db.k_cache
    v[:wl.num_blocks] = db.v_cache
    bt = wl.block_tables.copy()
    nxt = wl.num_blocks
    prefix = torch.from_numpy(bt[sharers[0], :64].astype(np.int64)).cuda()
    for s in sharers[1:]:
        ids = np.arange(nxt, nxt + 64)
        nxt += 64
        k[nxt - 64:nxt] = db.k_cache[prefix]
        v[nxt - 64:nxt] = db.v_cache[prefix]
        bt[s, :64] = ids
    db.k_cache, db.v_cache = k, v
    db.bt = torch.from_numpy(bt.astype(np.int32)).cuda()
    db.attend()
    torch.cuda.synchronize()
    private = to_host_bits(db.out)
    k2, v2 = oracle_after_append(wl)
    ref = oracle.paged_attention(wl.q, k2, v2, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                                 wl.num_kv_heads, wl.scale)
    compare(shared, ref, label="mixed-prefix-shared-layout")
    compare(private, ref, label="mixed-prefix-private-copies")
    # only block ids differ: without the sharing groups both layouts would take the same path
    # and agree bit for bit
    assert not np.array_equal(shared, private), "the shared layout did not take the group path"


def _share_case(name):
    """Batches whose decode rows share prefixes in the ways a radix prefix cache produces them."""
    rng = np.random.default_rng(len(name))
    if name == "share-two-groups-g4":
        specs = [(int(x), 1) for x in rng.integers(300, 2000, 40)]
        specs[3] = (300, 1)
        own = {21: 128, 22: 80, 23: 16, 24: 48}       # leave the prefix early (the last two: < one tile)
        share = [(list(range(0, 20)), 256), (list(range(20, 29)), 512, own)]
        return W.custom(name, specs, 32, 8, 128, 16, seed=1, share=share, row_order=rng.permutation(40))
    if name == "share-mha-d64-bs8":
        specs = [(int(x), 1) for x in rng.integers(1100, 1900, 24)]
        return W.custom(name, specs, 4, 4, 64, 8, seed=2, share=([i for i in range(24) if i % 6], 1024))
    if name == "share-g16":
        specs = [(int(x), 1) for x in rng.integers(700, 1500, 8)]
        return W.custom(name, specs, 16, 1, 128, 16, seed=3, share=([0, 2, 3, 5, 7], 640))
    if name == "share-g8-bs32-ragged":
        specs = [(int(x), 1) for x in rng.integers(2100, 3000, 9)]
        return W.custom(name, specs, 64, 8, 128, 32, seed=4, share=(list(range(7)), 2048))
    if name == "share-with-prefill-and-multirow":
        specs = [(int(x), 1) for x in rng.integers(900, 1600, 12)]
        specs += [(1200, 3), (1500, 2), (1200, 300), (1400, 64), (900, 1)]
        return W.custom(name, specs, 16, 4, 128, 16, seed=5, share=(list(range(16)), 832),
                        row_order=rng.permutation(len(specs)))
    if name == "share-long-prefix":
        specs = [(20000 + int(x), 1) for x in rng.integers(1, 4000, 10)]
        return W.custom(name, specs, 32, 8, 128, 16, seed=6, share=(list(range(10)), 20000))
    if name == "share-one-tile-members":
        specs = [(65, 1), (66, 1), (64, 1), (200, 1), (129, 1), (65, 1)]
        return W.custom(name, specs, 8, 2, 128, 16, seed=7, share=([0, 1, 2, 3, 4, 5], 64, {2: 48}))
    if name == "share-1000-sequences":
        # 8 KV heads per decode workgroup: detection runs up to 1024 sequences (16 per lane)
        specs = [(int(x), 1) for x in rng.integers(1025, 1600, 1000)]
        return W.custom(name, specs, 16, 8, 128, 16, seed=8, share=(list(range(0, 1000, 2)), 1024),
                        row_order=rng.permutation(1000))
    if name == "share-beyond-detection":
        # more sequences than detection covers (256 with 2 KV heads per workgroup): the rows
        # take the private path
        specs = [(70 + i % 7, 1) for i in range(4100)]
        return W.custom(name, specs, 8, 2, 128, 16, seed=9, share=(list(range(0, 4100, 3)), 64))
    raise KeyError(name)


def private_copies(db, wl):
    """Give every sequence its own copy of each block it shares with another (the pools are
    extended; the first sequence to reference a block keeps it).  Only block ids change, so
    the attention is the same; without sharing groups the kernels take the same path for
    both layouts and agree bit for bit."""
    import torch
    bt = wl.block_tables.copy()
    nblk = (wl.seq_lens.astype(np.int64) + wl.block_size - 1) // wl.block_size
    refs = {}
    for s in range(wl.num_seqs):
        for j in range(int(nblk[s])):
            refs[int(bt[s, j])] = refs.get(int(bt[s, j]), 0) + 1
    seen, moves, nxt = set(), [], wl.num_blocks
    for s in range(wl.num_seqs):
        for j in range(int(nblk[s])):
            b = int(bt[s, j])
            if refs[b] > 1 and b in seen:
                moves.append((nxt, b))
                bt[s, j] = nxt
                nxt += 1
            seen.add(b)
    k = torch.empty((nxt,) + tuple(db.k_cache.shape[1:]), dtype=db.k_cache.dtype, device=db.k_cache.device)
    v = torch.empty_like(k)
    k[:wl.num_blocks] = db.k_cache
    v[:wl.num_blocks] = db.v_cache
    if moves:
        dst = torch.tensor([m[0] for m in moves], device=k.device)
        src = torch.tensor([m[1] for m in moves], device=k.device)
        k[dst] = db.k_cache[src]
        v[dst] = db.v_cache[src]
    db.k_cache, db.v_cache = k, v
    db.bt = torch.from_numpy(bt.astype(np.int32)).to(k.device)
    return len(moves)


SHARE_CASES = ["share-two-groups-g4", "share-mha-d64-bs8", "share-g16", "share-g8-bs32-ragged",
               "share-with-prefill-and-multirow", "share-long-prefix", "share-one-tile-members",
               "share-1000-sequences", "share-beyond-detection"]


@pytest.mark.parametrize("name", SHARE_CASES)
def test_shared_prefix_groups(name):
    """Both layouts (shared blocks, and a private copy per sequence) against the oracle; the
    shared layout must take the group path (its output differs in rounding from the private
    layout's) except beyond the detection limit, where both take the same path."""
    wl = _share_case(name)
    print(f"{name}: {wl.num_seqs} sequences, groups {[len(g) for g in wl.meta['share_groups']]}", flush=True)
    db, shared, _ = run_and_check(wl, label=name)
    moved = private_copies(db, wl)
    db.attend()
    import torch
    torch.cuda.synchronize()
    private = to_host_bits(db.out)
    k2, v2 = oracle_after_append(wl)
    ref = oracle.paged_attention(wl.q, k2, v2, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                                 wl.num_kv_heads, wl.scale)
    compare(private, ref, label=name + "-private-copies")
    assert moved > 0
    if name == "share-beyond-detection":
        assert np.array_equal(shared, private)
    else:
        assert not np.array_equal(shared, private), "the shared layout did not take the group path"


def test_caller_workspace_and_stream(gpu):
    torch = gpu
    import paged_kv_cache_tables_amd as pkv
    wl = W.config1(num_seqs=8)
    db = DeviceBatch(wl)
    db.append()
    need = pkv.workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                               wl.max_blocks_per_seq, wl.block_size, wl.max_query_len)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        db.attend(workspace=ws)
    s.synchronize()
    got = to_host_bits(db.out)
    db.out.zero_()
    db.attend()
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(db.out), got)
    with pytest.raises(pkv.PagedKVError):
        db.attend(workspace=ws[: need - 256])


def test_library_workspace_on_a_side_stream(gpu):
    """A call on another stream without a caller workspace: the binding's own workspace comes
    from the current stream's memory pool and is released when the call returns, while the
    kernels may still run on the side stream.  Memory allocated and filled on the current
    stream right after the call must not land in that workspace (the result equals the
    same-stream result bit for bit)."""
    torch = gpu
    import paged_kv_cache_tables_amd as pkv
    wl = W.config1()
    db = DeviceBatch(wl)
    db.append()
    torch.cuda.synchronize()
    db.attend()
    torch.cuda.synchronize()
    want = to_host_bits(db.out)
    need = pkv.workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                               wl.max_blocks_per_seq, wl.block_size, wl.max_query_len)
    side = torch.cuda.Stream()
    for rep in range(3):
        db.out.zero_()
        torch.cuda.synchronize()
        pkv.paged_attention(db.out, db.q, db.k_cache, db.v_cache, db.bt, db.seq_lens, db.qsl, wl.scale,
                            wl.max_query_len, stream=side)
        junk = torch.empty(need, dtype=torch.uint8, device="cuda:0")
        junk.fill_(0x7F)                          # on the current stream, while the side stream may run
        torch.cuda.synchronize()
        del junk
        assert np.array_equal(to_host_bits(db.out), want), f"repetition {rep}"


def test_one_workspace_serves_calls_of_any_shape(gpu):
    """A workspace needs no initialisation and carries nothing between calls: one buffer,
    filled with junk before every call, serves calls of changing shape in turn."""
    torch = gpu
    import paged_kv_cache_tables_amd as pkv
    cases = [W.custom("ws-many", [(1 + (i * 53) % 3000, 1) for i in range(200)], 32, 8, 128, 16, seed=11),
             W.custom("ws-long", [(60000, 1), (5000, 1)], 16, 2, 128, 16, seed=12),
             W.custom("ws-multi", [(2000, 4), (700, 2), (300, 30)], 16, 4, 128, 16, seed=13),
             W.config1(num_seqs=16)]
    need = max(pkv.workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                   wl.max_blocks_per_seq, wl.block_size, wl.max_query_len) for wl in cases)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    for rnd in range(2):
        for wl in cases:
            print(f"shared workspace: {wl.name} round {rnd}", flush=True)
            db = DeviceBatch(wl)
            db.append()
            ws.fill_(0x5A + rnd)
            db.attend(workspace=ws)
            torch.cuda.synchronize()
            k2, v2 = oracle_after_append(wl)
            ref = oracle.paged_attention(wl.q, k2, v2, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                                         wl.num_kv_heads, wl.scale)
            compare(to_host_bits(db.out), ref, label=f"shared-ws-{wl.name}")


@pytest.mark.parametrize("cfg", [0, 1, "share", 3, "split"])
def test_step_captured_in_hip_graph(gpu, cfg):
    """append + attention captured once in a HIP graph (the library allocates, memsets and
    synchronises nothing inside a call), replayed with new queries written in between by
    eager work: every replay equals the eager call on the same inputs, bit for bit."""
    torch = gpu
    import paged_kv_cache_tables_amd as pkv
    print(f"graph capture config {cfg}", flush=True)
    # config 3 and "share": decode rows in sharing groups (found from the tables in every
    # replay), config 3 also prefill rows and the planner; "split": a chunk over a long prefix,
    # its items cut into pieces whose counters the planner clears in every replay
    wl = {0: lambda: W.config0(), 1: lambda: W.config1(num_seqs=16), 3: lambda: W.config3(),
          "share": lambda: _share_case("share-two-groups-g4"),
          "split": lambda: W.custom("graph-split", [(20000 + 64, 64), (3000, 1), (500, 1)], 32, 8, 128, 16,
                                    seed=21)}[cfg]()
    db = DeviceBatch(wl)
    need = pkv.workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                               wl.max_blocks_per_seq, wl.block_size, wl.max_query_len)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    q_alt = [db.q.clone(), torch.flip(db.q, dims=[1]).contiguous(), (db.q * 0.5).contiguous()]

    def eager(qv):
        db.q.copy_(qv)
        db.append()
        db.attend(workspace=ws)
        torch.cuda.synchronize()
        return to_host_bits(db.out)

    want = [eager(qv) for qv in q_alt]
    # the eager result itself is the oracle's (first query set)
    k2, v2 = oracle_after_append(wl)
    ref = oracle.paged_attention(wl.q, k2, v2, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                                 wl.num_kv_heads, wl.scale)
    compare(want[0], ref, label=f"graph-eager-{cfg}")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        db.append()
        db.attend(workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        db.append()
        db.attend(workspace=ws)
    torch.cuda.synchronize()
    for rep in range(6):
        i = rep % len(q_alt)
        db.q.copy_(q_alt[i])
        db.out.zero_()
        ws.fill_(0xA5)            # stale partials from another call must not leak into this one
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(db.out), want[i]), f"replay {rep} (query set {i}) differs"
