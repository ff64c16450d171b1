"""GPU check of paged_attention_append_noalloc, the entry point that allocates nothing.

It is paged_attention_append with the split-K partials in the library's static per-GPU
scratch instead of a caller workspace.  Called through the C ABI, it must leave the pools
and the output exactly as paged_attention_append does (bit for bit: same kernels, same
order of operations), on two calls in a row, the second with a smaller batch (the scratch
keeps the first call's contents, which must not leak into the second), and reject a shape
that needs more than the scratch holds without enqueueing anything.
"""
import numpy as np
import pytest

import workloads as W
from gpu_harness import DeviceBatch, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import paged_kv_cache_tables_amd as pkv
    pkv.load_library()
    return torch


def _pair(wl):
    """Two device copies of the batch: one for each entry point."""
    return DeviceBatch(wl), DeviceBatch(wl)


def _fused(pkv, db, noalloc):
    args = (db.out, db.q, db.k_new, db.v_new, db.slots, db.k_cache, db.v_cache, db.bt, db.seq_lens, db.qsl,
            db.wl.scale, db.wl.max_query_len)
    if noalloc:
        pkv.paged_attention_append_noalloc(*args)
    else:
        pkv.paged_attention_append(*args)


def test_noalloc_equals_workspace_call_twice_shrinking(gpu):
    torch = gpu
    import paged_kv_cache_tables_amd as pkv
    cases = [W.config3(), W.config1(num_seqs=24)]      # the second call's batch is smaller
    for i, wl in enumerate(cases):
        print(f"noalloc call {i}: {wl.name}, {wl.num_seqs} sequences", flush=True)
        ref, got = _pair(wl)
        _fused(pkv, ref, noalloc=False)
        _fused(pkv, got, noalloc=True)
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(got.k_cache), to_host_bits(ref.k_cache)), "K pool differs"
        assert np.array_equal(to_host_bits(got.v_cache), to_host_bits(ref.v_cache)), "V pool differs"
        assert np.array_equal(to_host_bits(got.out), to_host_bits(ref.out)), "output differs"


def test_noalloc_split_prefill_twice(gpu):
    """Chunks over long prefixes whose items are cut into pieces: the pieces' partials and the
    per-item counters that find the last piece live in the scratch too, and the planner clears
    the counters it uses on every call (the second call reuses slots the first one raised)."""
    torch = gpu
    import paged_kv_cache_tables_amd as pkv
    cases = [W.custom("noalloc-split-a", [(20000 + 64, 64), (3000, 1), (500, 1)], 32, 8, 128, 16, seed=11),
             W.custom("noalloc-split-b", [(9000 + 40, 40)], 32, 8, 128, 16, seed=12)]
    for i, wl in enumerate(cases):
        print(f"noalloc split call {i}: {wl.name}, {wl.num_q_tokens} rows", flush=True)
        ref, got = _pair(wl)
        _fused(pkv, ref, noalloc=False)
        _fused(pkv, got, noalloc=True)
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(got.k_cache), to_host_bits(ref.k_cache)), "K pool differs"
        assert np.array_equal(to_host_bits(got.out), to_host_bits(ref.out)), "output differs"


def test_noalloc_long_context_and_too_large_shape(gpu):
    torch = gpu
    import paged_kv_cache_tables_amd as pkv
    wl = W.config4(num_seqs=2)
    print(f"noalloc: {wl.name}, {wl.num_seqs} sequences", flush=True)
    ref, got = _pair(wl)
    _fused(pkv, ref, noalloc=False)
    _fused(pkv, got, noalloc=True)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(got.out), to_host_bits(ref.out)), "output differs"
    # a shape that needs more than the scratch (its prefill work list: 256 sequences of up to
    # 2^20 tokens): rejected before anything is enqueued, nothing written
    T, Hq, Hkv, D, max_blocks = 256, 32, 8, 128, 65536
    need = pkv.workspace_bytes(T, Hq, Hkv, D, max_blocks, 16, 2)
    assert need > pkv.NOALLOC_SCRATCH_BYTES
    dev = "cuda:0"
    q = torch.zeros((T, Hq, D), dtype=torch.bfloat16, device=dev)
    out = torch.full_like(q, 1.0)
    kn = torch.zeros((T, Hkv, D), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((64, 16, Hkv, D), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    bt = torch.zeros((T, max_blocks), dtype=torch.int32, device=dev)
    sl = torch.full((T,), 2, dtype=torch.int32, device=dev)
    qsl = torch.arange(T + 1, dtype=torch.int32, device=dev)
    slots = torch.arange(T, dtype=torch.int64, device=dev)
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_attention_append_noalloc(out, q, kn, kn, slots, kc, vc, bt, sl, qsl, 0.088, 2)
    assert e.value.status == -6
    torch.cuda.synchronize()
    assert (kc == 0).all() and (out == 1.0).all()
