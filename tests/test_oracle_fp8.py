"""Pins of the FP8 (E4M3) oracle: code values, nearest-even quantisation, the
append and attention over dequantised pools -- each against something other
than the oracle itself (values fixed by the format's field definitions,
torch's float8_e4m3fn conversion, closed forms and the bf16 attention oracle)."""
import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")


def torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_encode(y):
    return torch.from_numpy(np.asarray(y, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# -- code values ---------------------------------------------------------------

@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0),
    (0x3F, 1.875), (0x40, 2.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0), (0x81, -(2.0 ** -9)),
])
def test_named_codes(code, value):
    assert oracle.e4m3_value(code) == value


def test_nan_codes_and_signed_zero():
    assert np.isnan(oracle.e4m3_value(0x7F)) and np.isnan(oracle.e4m3_value(0xFF))
    assert np.signbit(oracle.e4m3_value(0x80)) and oracle.e4m3_value(0x80) == 0.0


def test_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = oracle.e4m3_to_f64(codes), torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


# -- quantisation --------------------------------------------------------------

def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    y = np.concatenate([rng.standard_normal(20000) * s for s in (2.0 ** -8, 2.0 ** -4, 1.0, 16.0, 100.0)])
    y = y[np.abs(y) <= 464.0].astype(np.float32)
    assert np.array_equal(oracle.f64_to_e4m3(y.astype(np.float64)), torch_encode(y))


def test_encode_midpoints_round_to_even():
    vals = oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))   # 0 .. 448, increasing
    mids = (vals[:-1] + vals[1:]) / 2                             # exact in float64 (and float32)
    got = oracle.f64_to_e4m3(mids)
    lo = np.arange(0x7E, dtype=np.uint8)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    assert np.array_equal(got, torch_encode(mids.astype(np.float32)))
    assert np.array_equal(oracle.f64_to_e4m3(-mids), want | 0x80)


def test_encode_round_trip_and_monotone():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oracle.f64_to_e4m3(oracle.e4m3_to_f64(codes)), codes)
    y = np.linspace(0, 460, 200001)
    c = oracle.f64_to_e4m3(y).astype(np.int64)
    assert (np.diff(c) >= 0).all()


def test_encode_saturates():
    y = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e6, -1e6, -500.0])
    assert oracle.f64_to_e4m3(y).tolist() == [0x7E] * 6 + [0xFE, 0xFE]


def test_encode_error_bound():
    # nearest rounding: |decode(encode(y)) - y| <= half the gap to the neighbouring value
    rng = np.random.default_rng(3)
    y = rng.uniform(-448, 448, 50000)
    err = np.abs(oracle.e4m3_to_f64(oracle.f64_to_e4m3(y)) - y)
    mag = np.abs(y)
    e = np.floor(np.log2(np.maximum(mag, 2.0 ** -6)))
    half_gap = 2.0 ** (e - 3) / 2
    assert (err <= half_gap * (1 + 1e-12)).all()


@pytest.mark.parametrize("scale,bits", [
    (0.75, [0x3F80, 0x3FC0, 0xC030, 0x4396]),
    # inputs whose float32 quotient is rounded onto (or off) a midpoint of two codes, so that
    # the float32 and the exact quotient give different codes
    # (the exact quotient by the float32 scale, the quotient by the unrounded scale, or the
    # product with a float32 reciprocal)
    (0.1, [0x3AC0]), (0.7, [0x3B60, 0x3C8C, 0x3D0C, 0x3D8C]), (1 / 3, [0x3A80, 0x3BA0, 0x3C10, 0x3C90]),
    (0.3, [0x3B90]), (0.6, [0x3C10]), (0.9, [0x3B90, 0x3CB4, 0x3D34, 0x3DB4]),
])
def test_quantize_uses_float32_quotient(scale, bits):
    x = np.array(bits, dtype=np.uint16)
    codes = oracle.quantize_bf16(x, scale)
    y = (x.astype(np.uint32) << 16).view(np.float32) / np.float32(scale)
    assert np.array_equal(codes, torch_encode(y))


# -- append --------------------------------------------------------------------

def test_append_fp8_writes_codes_and_leaves_the_rest():
    wl = W.config0()
    k0 = np.full((wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim), 0x7F, np.uint8)
    v0 = k0.copy()
    slots = wl.slot_mapping.copy()
    slots[2] = -1
    k1, v1 = oracle.kv_append_fp8(k0, v0, wl.k_new, wl.v_new, slots, 0.125, 0.5)
    bs = wl.block_size
    for i, s in enumerate(slots):
        if s < 0:
            continue
        xk = (wl.k_new[i].astype(np.uint32) << 16).view(np.float32) / np.float32(0.125)
        xv = (wl.v_new[i].astype(np.uint32) << 16).view(np.float32) / np.float32(0.5)
        assert np.array_equal(k1[s // bs, s % bs], torch_encode(xk))
        assert np.array_equal(v1[s // bs, s % bs], torch_encode(xv))
    touched = np.zeros(k0.shape[:2], bool)
    for s in slots[slots >= 0]:
        touched[s // bs, s % bs] = True
    assert (k1[~touched] == 0x7F).all() and (v1[~touched] == 0x7F).all()


def test_append_fp8_rejects_bad_scale_and_slots():
    wl = W.config0()
    k0 = np.zeros((wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim), np.uint8)
    with pytest.raises(ValueError):
        oracle.kv_append_fp8(k0, k0, wl.k_new, wl.v_new, wl.slot_mapping, 0.0, 1.0)
    bad = wl.slot_mapping.copy()
    bad[1] = bad[0]
    with pytest.raises(ValueError):
        oracle.kv_append_fp8(k0, k0, wl.k_new, wl.v_new, bad, 1.0, 1.0)


# -- attention over dequantised pools ------------------------------------------

def _bf16_pool_of(codes, scale_pow2):
    """bf16 bits of code_value * 2^k (exact: E4M3 values scaled by a power of two are bf16 values)."""
    f = (torch_decode(codes) * scale_pow2).astype(np.float32)
    f = np.where(np.isnan(f), np.float32(np.nan), f)
    return W.f32_to_bf16_bits(f)


@pytest.mark.parametrize("variant", ["A", "B"])
def test_attention_fp8_equals_bf16_attention_on_exact_values(variant):
    wl = W.config0(variant=variant)
    f8 = W.fp8_pools(wl)
    ks, vs = f8.k_scale, f8.v_scale
    k2, v2 = oracle.kv_append_fp8(f8.k_cache, f8.v_cache, wl.k_new, wl.v_new, wl.slot_mapping, ks, vs)
    got = oracle.paged_attention_fp8(wl.q, k2, v2, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                                     wl.num_kv_heads, wl.scale, ks, vs)
    ref = oracle.paged_attention(wl.q, _bf16_pool_of(k2, ks), _bf16_pool_of(v2, vs), wl.block_tables,
                                 wl.seq_lens, wl.query_start_loc, wl.num_kv_heads, wl.scale)
    assert np.array_equal(got, ref)


def test_attention_fp8_length_one_is_the_value_row():
    wl = W.config0()
    f8 = W.fp8_pools(wl)
    k2, v2 = oracle.kv_append_fp8(f8.k_cache, f8.v_cache, wl.k_new, wl.v_new, wl.slot_mapping,
                                  f8.k_scale, f8.v_scale)
    out = oracle.paged_attention_fp8(wl.q, k2, v2, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                                     wl.num_kv_heads, wl.scale, f8.k_scale, f8.v_scale)
    # sequence 0 has one token: out = its dequantised V row for every head of its group
    G = wl.num_q_heads // wl.num_kv_heads
    s = int(wl.slot_mapping[0])
    bs = wl.block_size
    for g in range(wl.num_q_heads):
        want = torch_decode(v2[s // bs, s % bs, g // G]) * np.float64(np.float32(f8.v_scale))
        assert np.array_equal(out[0, g], want)


def test_attention_fp8_ignores_poisoned_slots():
    wl = W.config0()
    a = W.fp8_pools(wl, poison=0x7F)
    b = W.fp8_pools(wl, poison=0xFF)
    outs = []
    for f8 in (a, b):
        k2, v2 = oracle.kv_append_fp8(f8.k_cache, f8.v_cache, wl.k_new, wl.v_new, wl.slot_mapping,
                                      f8.k_scale, f8.v_scale)
        outs.append(oracle.paged_attention_fp8(wl.q, k2, v2, wl.block_tables, wl.seq_lens,
                                               wl.query_start_loc, wl.num_kv_heads, wl.scale,
                                               f8.k_scale, f8.v_scale))
    assert np.isfinite(outs[0]).all() and np.array_equal(outs[0], outs[1])
