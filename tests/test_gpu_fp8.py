"""GPU parity of the 8-bit (E4M3) cache: the HIP library through the C ABI
against the float64 CPU oracle.

Bars: kv_append_fp8 is bit-exact (codes) over the whole pool; attention over
8-bit pools has the bf16 pools' tolerance against the oracle's attention of
the dequantised values (1e-2 max abs, raised to one bf16 ulp of the reference
where that is larger, and 1e-3 mean abs): the kernels widen codes exactly, so
only the bf16 output rounding and fp32 accumulation differ.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_harness import compare, to_dev, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import paged_kv_cache_tables_amd as pkv
    pkv.load_library()
    return torch


class DeviceBatchFp8:
    """Device copies of a workload with 8-bit pools (before the append)."""

    def __init__(self, wl, f8, device="cuda:0"):
        import torch
        self.wl, self.f8 = wl, f8
        self.q = to_dev(wl.q, torch.bfloat16, device)
        self.k_new = to_dev(wl.k_new, torch.bfloat16, device)
        self.v_new = to_dev(wl.v_new, torch.bfloat16, device)
        self.slots = to_dev(wl.slot_mapping.astype(np.int64), torch.int64, device)
        self.k_cache = torch.from_numpy(f8.k_cache).to(device)
        self.v_cache = torch.from_numpy(f8.v_cache).to(device)
        self.bt = to_dev(wl.block_tables.astype(np.int32), torch.int32, device)
        self.seq_lens = to_dev(wl.seq_lens.astype(np.int32), torch.int32, device)
        self.qsl = to_dev(wl.query_start_loc.astype(np.int32), torch.int32, device)
        self.out = torch.empty_like(self.q)

    def append(self):
        import paged_kv_cache_tables_amd as pkv
        pkv.kv_append_fp8(self.k_new, self.v_new, self.slots, self.k_cache, self.v_cache,
                          self.f8.k_scale, self.f8.v_scale)

    def attend(self):
        import paged_kv_cache_tables_amd as pkv
        pkv.paged_attention_fp8(self.out, self.q, self.k_cache, self.v_cache, self.bt, self.seq_lens,
                                self.qsl, self.wl.scale, self.wl.max_query_len, self.f8.k_scale,
                                self.f8.v_scale)

    def step(self):
        self.append()
        self.attend()


def oracle_pools(wl, f8):
    return oracle.kv_append_fp8(f8.k_cache, f8.v_cache, wl.k_new, wl.v_new, wl.slot_mapping,
                                f8.k_scale, f8.v_scale)


def run_and_check(wl, f8=None, rows=None, label=""):
    import torch
    f8 = f8 or W.fp8_pools(wl)
    print(f"fp8 case {label or wl.name}", flush=True)
    db = DeviceBatchFp8(wl, f8)
    db.step()
    torch.cuda.synchronize()
    k2, v2 = oracle_pools(wl, f8)
    assert np.array_equal(db.k_cache.cpu().numpy(), k2) and np.array_equal(db.v_cache.cpu().numpy(), v2)
    ref = oracle.paged_attention_fp8(wl.q, k2, v2, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                                     wl.num_kv_heads, wl.scale, f8.k_scale, f8.v_scale, rows=rows)
    return compare(to_host_bits(db.out), ref, rows=rows, label=label or wl.name)


# ---------------------------------------------------------------------------
# append: codes bit-exact over the whole pool
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_append_fp8_bit_exact_whole_pool(cfg):
    import torch
    print(f"fp8 append config {cfg}", flush=True)
    wl = W.make_config(cfg)
    f8 = W.fp8_pools(wl)
    db = DeviceBatchFp8(wl, f8)
    db.append()
    torch.cuda.synchronize()
    k2, v2 = oracle_pools(wl, f8)
    assert np.array_equal(db.k_cache.cpu().numpy(), k2)
    assert np.array_equal(db.v_cache.cpu().numpy(), v2)


def test_append_fp8_rounding_ties_subnormals_and_saturation():
    """New rows whose quotients hit exact midpoints between codes, subnormals, zeros of
    both signs, values past the largest code, and quotients whose float32 rounding
    decides the code."""
    import torch
    wl = W.custom("fp8-edges", [(40, 8), (9, 1)], 4, 2, 128, 16, seed=5)
    vals = oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2                               # exact ties
    extra = np.array([0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -11, 448.0, 460.0, 464.0, 470.0, 1e4, 3e38])
    pool = np.concatenate([mids, -mids, vals, extra, -extra])
    k_scale, v_scale = 2.0 ** -4, 0.7
    kv = np.resize(pool, wl.k_new.size).reshape(wl.k_new.shape)
    # K: quotient by a power of two is exact, so the ties are exact ties of y
    wl.k_new = W.f32_to_bf16_bits((kv * k_scale).astype(np.float32))
    # V: bf16 values whose float32 quotient by 0.7 lands on or off a midpoint
    vbits = np.array([0x3B60, 0x3C8C, 0x3D0C, 0x3D8C, 0xBB60, 0x4396, 0x3F80, 0x0001], dtype=np.uint16)
    wl.v_new = np.resize(vbits, wl.v_new.size).reshape(wl.v_new.shape)
    f8 = W.fp8_pools(wl, k_scale=k_scale, v_scale=v_scale)
    db = DeviceBatchFp8(wl, f8)
    db.append()
    torch.cuda.synchronize()
    k2, v2 = oracle_pools(wl, f8)
    assert np.array_equal(db.k_cache.cpu().numpy(), k2)
    assert np.array_equal(db.v_cache.cpu().numpy(), v2)


def test_append_fp8_skips_padding_and_keeps_poison():
    import torch
    wl = W.config0()
    wl.slot_mapping = wl.slot_mapping.copy()
    wl.slot_mapping[[0, 5]] = -1
    f8 = W.fp8_pools(wl, poison=0xFF)
    db = DeviceBatchFp8(wl, f8)
    db.append()
    torch.cuda.synchronize()
    k2, v2 = oracle_pools(wl, f8)
    assert np.array_equal(db.k_cache.cpu().numpy(), k2)
    assert np.array_equal(db.v_cache.cpu().numpy(), v2)


# ---------------------------------------------------------------------------
# attention parity on the five configurations
# ---------------------------------------------------------------------------

def test_fp8_config0_all_rows_and_length_one_exact():
    wl = W.config0()
    f8 = W.fp8_pools(wl)
    run_and_check(wl, f8)
    import torch
    db = DeviceBatchFp8(wl, f8)
    db.step()
    torch.cuda.synchronize()
    # sequence 0 has one token: bf16 of its dequantised V row (value x 2^-3, exact in bf16)
    G = wl.num_q_heads // wl.num_kv_heads
    s, bs = int(wl.slot_mapping[0]), wl.block_size
    k2, v2 = oracle_pools(wl, f8)
    want = W.f32_to_bf16_bits((oracle.e4m3_to_f64(v2[s // bs, s % bs]) * f8.v_scale).astype(np.float32))
    out = to_host_bits(db.out)
    for g in range(wl.num_q_heads):
        assert np.array_equal(out[0, g], want[g // G])


def test_fp8_config0_variant_b():
    run_and_check(W.config0(variant="B"))


def test_fp8_config1_decode_all_rows():
    run_and_check(W.config1())


def test_fp8_config2_decode_all_rows():
    run_and_check(W.config2())


def test_fp8_config3_mixed_all_rows():
    run_and_check(W.config3())


def test_fp8_config4_long_context_all_rows():
    run_and_check(W.config4())


# ---------------------------------------------------------------------------
# shapes, scales and edge cases
# ---------------------------------------------------------------------------

EDGE8 = [
    # name, seq_specs (L, q), Hq, Hkv, D, bs
    ("f8-bs8-d128-g4", [(1, 1), (9, 1), (700, 1), (130, 3), (300, 300)], 8, 2, 128, 8),
    ("f8-bs32-d128-g8", [(33, 1), (1025, 1), (2000, 64), (64, 64)], 16, 2, 128, 32),
    ("f8-d64-g1-mha", [(5, 1), (513, 1), (100, 37), (1, 1)], 4, 4, 64, 16),
    ("f8-d64-g16-bs32", [(17, 1), (4000, 1), (200, 150)], 16, 1, 64, 32),
    ("f8-split-tails", [(511, 1), (512, 1), (513, 1), (1024, 1), (1025, 1), (65, 1)], 8, 2, 128, 16),
    ("f8-long-many-pieces", [(60000, 1), (3, 1)], 8, 2, 128, 16),
    ("f8-multi-row-g4", [(700, 4), (5, 2), (1300, 3), (64, 4), (900, 1)], 16, 4, 128, 16),
    ("f8-short-and-long-chunks", [(800, 4), (1000, 300), (2000, 1), (90, 3), (513, 64)], 32, 8, 128, 16),
    ("f8-chunk-from-zero", [(512, 512), (97, 97)], 32, 8, 128, 16),
    # a chunk over a long prefix: items cut into pieces of key tiles, partials merged
    ("f8-split-long-prefix", [(20000 + 64, 64), (3000, 1)], 32, 8, 128, 16),
    ("f8-split-d64-mha", [(12000 + 128, 128)], 8, 8, 64, 16),
]


@pytest.mark.parametrize("name,specs,Hq,Hkv,D,bs", EDGE8, ids=[e[0] for e in EDGE8])
def test_fp8_edge_shapes(name, specs, Hq, Hkv, D, bs):
    wl = W.custom(name, specs, Hq, Hkv, D, bs, seed=len(name))
    run_and_check(wl)


@pytest.mark.parametrize("k_scale,v_scale", [(0.011, 0.37), (2.0 ** -7, 2.0 ** 2)])
def test_fp8_non_power_of_two_and_wide_scales(k_scale, v_scale):
    wl = W.custom("f8-scales", [(300, 1), (1200, 1), (400, 90)], 16, 4, 128, 16, seed=11)
    run_and_check(wl, W.fp8_pools(wl, k_scale=k_scale, v_scale=v_scale), label=f"scales {k_scale} {v_scale}")


def test_fp8_poisoned_slots_do_not_change_the_output():
    import torch
    outs = []
    for poison in (0x7F, 0xFF, 0x00, 0x7E):
        wl = W.custom("f8-poison", [(70, 1), (300, 45), (1500, 1), (5, 1)], 8, 2, 128, 16, seed=9)
        db = DeviceBatchFp8(wl, W.fp8_pools(wl, poison=poison))
        db.step()
        torch.cuda.synchronize()
        outs.append(to_host_bits(db.out))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_fp8_run_to_run_determinism():
    import torch
    wl = W.config3()
    db = DeviceBatchFp8(wl, W.fp8_pools(wl))
    db.step()
    torch.cuda.synchronize()
    first = to_host_bits(db.out)
    for _ in range(2):
        db.attend()
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(db.out), first)
