"""Host-side checks of the seeded workload generator (shapes and stated readings)."""
import numpy as np

import workloads as W


def _common_checks(wl):
    T = wl.num_q_tokens
    assert wl.q.shape == (T, wl.num_q_heads, wl.head_dim)
    assert wl.k_new.shape == wl.v_new.shape == (T, wl.num_kv_heads, wl.head_dim)
    assert wl.query_start_loc[0] == 0 and wl.query_start_loc[-1] == T
    assert (np.diff(wl.query_start_loc) >= 0).all()
    assert (wl.query_lens <= wl.seq_lens).all()
    # new tokens go to unique, private, in-pool slots
    assert len(np.unique(wl.slot_mapping)) == T
    assert (wl.slot_mapping >= 0).all() and (wl.slot_mapping < wl.num_blocks * wl.block_size).all()
    # cached slots are unique and disjoint from the new ones
    assert len(np.unique(wl.cached_slots)) == wl.cached_slots.size
    assert not np.isin(wl.slot_mapping, wl.cached_slots).any()
    # table entries in range where used, -1 elsewhere
    for s in range(wl.num_seqs):
        nb = (int(wl.seq_lens[s]) + wl.block_size - 1) // wl.block_size
        assert (wl.block_tables[s, :nb] >= 0).all() and (wl.block_tables[s, :nb] < wl.num_blocks).all()
        assert (wl.block_tables[s, nb:] == -1).all()


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 65504.0, np.inf, -np.inf, np.nan], np.float32)
    got = W.f32_to_bf16_bits(x)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6)
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x4780, 0x7F80, 0xFF80, 0x7FC0]


def test_config0_reading_a_and_b():
    a = W.config0()
    _common_checks(a)
    assert a.seq_lens.tolist() == [1, 7, 16, 38]
    assert a.query_lens.tolist() == [1, 1, 1, 5]
    assert a.num_blocks == 64 and a.scale == 0.125
    b = W.config0(variant="B")
    _common_checks(b)
    assert b.seq_lens.tolist() == [1, 7, 21, 33]
    assert b.query_lens.tolist() == [1, 1, 5, 1]


def test_config0_pool_poisoned_except_cached():
    a = W.config0()
    flat = a.k_cache.reshape(-1, a.num_kv_heads, a.head_dim)
    mask = np.zeros(flat.shape[0], bool)
    mask[a.cached_slots] = True
    assert (flat[~mask] == W.BF16_QNAN).all()
    assert not (flat[mask] == W.BF16_QNAN).any()


def test_config3_prefix_sharing_reading():
    wl = W.config3()
    _common_checks(wl)
    sharers = wl.meta["sharers"]
    assert len(sharers) == 100
    first = wl.block_tables[sharers[0], :64]
    for s in sharers:
        assert np.array_equal(wl.block_tables[s, :64], first)
    ql = wl.query_lens
    assert sorted(ql[ql > 1].tolist()) == [512] * 8
    assert (ql >= 1).all() and int((ql == 1).sum()) == 192
    # prefill and decode rows are interleaved in the batch order
    kinds = (ql > 1).astype(int)
    assert 0 < np.nonzero(kinds)[0].min() or np.nonzero(kinds)[0].max() < len(kinds) - 1
    # unique bytes count the 64 shared blocks once
    saved = (len(sharers) - 1) * 64 * 16 * 2 * 8 * 128 * 2
    assert wl.kv_read_bytes() - wl.unique_kv_read_bytes() == saved


def test_config4_outliers_are_one_percent_per_head():
    L = 2000
    wl = W.config4(ctx=L, num_seqs=2)
    base = W.config4(ctx=L, num_seqs=2, outlier_frac=0.0)
    _common_checks(wl)
    for s in range(2):
        # logical K rows of sequence s, from its cached rows (in slot order) and its new row
        sl = slice(s * (L - 1), (s + 1) * (L - 1))
        k = np.concatenate([wl.cached_k[sl], wl.k_new[s:s + 1]])
        k0 = np.concatenate([base.cached_k[sl], base.k_new[s:s + 1]])
        f = (k.astype(np.uint32) << 16).view(np.float32)
        f0 = (k0.astype(np.uint32) << 16).view(np.float32)
        changed = (k != k0).any(axis=2)                       # [L, Hkv]
        assert (changed.sum(axis=0) == L // 100).all()        # floor(0.01 L) rows per head
        assert np.array_equal(f[changed], 8.0 * f0[changed])  # whole row x8, exact
        assert np.array_equal(wl.v_new, base.v_new)           # V untouched


def test_seed_determinism_and_placement_independence():
    a = W.config0(seed=5)
    b = W.config0(seed=5)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k_cache, b.k_cache)
    c = W.config0(seed=5, placement_seed=99)
    assert np.array_equal(a.q, c.q) and np.array_equal(a.k_new, c.k_new)
    assert not np.array_equal(a.block_tables, c.block_tables)
