"""Plain float64 reference of the FP8 KV cache (test infrastructure only).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT (see the package docstring).

Sources (web pages; cited by title and section):
  [SPEED] "How to Speed Up LLM Inference: KV Cache to Production Serving"
          (fatherofai) -- "The KV cache: the memory problem that runs the show"
          (quantising the cache itself to FP8 halves the bytes per token) and
          "Quantization: move fewer bytes" (values stored in few bits with a
          shared scale factor and multiplied after dequantisation in registers:
          the gain is bandwidth only).
  [TGI]   "Text Generation Inference: ..." -- "Production Pattern: KV Cache
          Math" (the FP8 row of the bytes-per-token table: one byte per value).

Readings where the pages are silent:
  * The 8-bit format is E4M3 in the encoding without infinities ("FN"): sign
    bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
    the subnormals m * 2^-9; the all-ones pattern S.1111.111 is NaN; the
    largest finite magnitude is 448.
  * One float32 scale per pool (one for K, one for V), chosen by the caller:
    the cache holds exactly one byte per value, as the pages' "halves the
    bytes" figure implies.  A cached value stands for code_value * scale.
  * Quantising a bf16 value x: y = float32(x) / float32(scale), the float32
    quotient correctly rounded; then the E4M3 value nearest to y, ties to the
    even code (mantissa bit 0 clear); |y| beyond the nearest-rounding range
    gives the largest finite value of its sign (saturation, never NaN).
  * Attention over an FP8 cache is the exact softmax attention of the
    dequantised values code_value * scale (in float64).
"""
from __future__ import annotations

import numpy as np

from .paged import bf16_bits_to_f64, gather_tokens, kv_head_of, row_position, softmax_attend

E4M3_BIAS = 7
E4M3_MAX_CODE = 0x7E          # 448: exponent field 15, mantissa 6
E4M3_NAN = 0x7F


def e4m3_value(code: int) -> float:
    """Value of one E4M3 (FN) code, from the field definitions."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = m * 2.0 ** (1 - E4M3_BIAS - 3)          # subnormal: (m / 8) * 2^(1 - bias)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - E4M3_BIAS)
    return sign * mag


# value of every code, once
_VALUES = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# the non-negative finite values, increasing with the code (codes 0x00 .. 0x7E)
_POS = _VALUES[:E4M3_MAX_CODE + 1]


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode an array of E4M3 codes (uint8) exactly."""
    return _VALUES[np.asarray(codes, dtype=np.uint8)]


def f64_to_e4m3(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code to each finite y, ties to the even code, saturating at +-448.

    The magnitude is placed between two consecutive non-negative values of the
    format; the nearer one wins and an exact midpoint takes the code whose
    mantissa bit 0 is clear.  The sign is copied (a negative value that rounds
    to zero gives the code of -0).
    """
    y = np.asarray(y, dtype=np.float64)
    if not np.isfinite(y).all():
        raise ValueError("only finite values are quantised")
    mag = np.abs(y)
    hi = np.searchsorted(_POS, mag, side="left")            # first value >= mag
    hi = np.minimum(hi, E4M3_MAX_CODE)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS[lo]
    d_hi = _POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(mag >= _POS[E4M3_MAX_CODE], E4M3_MAX_CODE, code)   # saturate
    code = np.where(mag == 0.0, 0, code)
    sign = np.signbit(y)
    return (code.astype(np.uint16) | np.where(sign, 0x80, 0)).astype(np.uint8)


def quantize_bf16(bits: np.ndarray, scale: float) -> np.ndarray:
    """E4M3 codes of bf16 values divided by ``scale`` (float32 quotient, then nearest code)."""
    x = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    y = x / np.float32(scale)                                  # IEEE float32 division
    return f64_to_e4m3(y.astype(np.float64))


def kv_append_fp8(k_cache, v_cache, k_new, v_new, slot_mapping, k_scale: float, v_scale: float):
    """Quantise each new token's K and V rows and write the codes into its slot.

    The slot rules are those of the bf16 append ([TGI] "Under the Hood:
    PagedAttention"; slot = block * block_size + offset; slot < 0 is padding,
    an out-of-pool or repeated slot is an error).  Pools are uint8 code arrays
    [NB, bs, Hkv, D]; returns new pools.
    """
    k_out = np.array(k_cache, dtype=np.uint8, copy=True)
    v_out = np.array(v_cache, dtype=np.uint8, copy=True)
    NB, bs = k_out.shape[0], k_out.shape[1]
    slots = np.asarray(slot_mapping, dtype=np.int64)
    if k_new.shape[0] != slots.shape[0] or v_new.shape[0] != slots.shape[0]:
        raise ValueError("one slot per new token")
    if not (np.isfinite(np.float32(k_scale)) and np.float32(k_scale) > 0 and
            np.isfinite(np.float32(v_scale)) and np.float32(v_scale) > 0):
        raise ValueError("scales must be positive and finite")
    live = slots[slots >= 0]
    if live.size and live.max() >= NB * bs:
        raise ValueError("slot outside the pool")
    if np.unique(live).size != live.size:
        raise ValueError("duplicate slot in one append")
    kq = quantize_bf16(k_new, k_scale)
    vq = quantize_bf16(v_new, v_scale)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        k_out[int(slot) // bs, int(slot) % bs] = kq[i]
        v_out[int(slot) // bs, int(slot) % bs] = vq[i]
    return k_out, v_out


def paged_attention_fp8(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
                        num_kv_heads: int, scale: float, k_scale: float, v_scale: float,
                        rows=None) -> np.ndarray:
    """The attention of ``oracle.paged_attention`` over FP8 pools.

    Each gathered key and value row is dequantised as code_value * scale (the
    float32 scales widened to float64), then the definition is evaluated as
    for bf16 pools: row j of sequence s at position L - q_s + j attends keys
    0..that position of KV head g // (Hq / Hkv).  Returns float64.
    """
    q = np.asarray(q, dtype=np.uint16)
    T, Hq, D = q.shape
    Hkv = int(num_kv_heads)
    group = Hq // Hkv
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    L_all = np.asarray(seq_lens, dtype=np.int64)
    bt = np.asarray(block_tables)
    scale64 = float(np.float32(scale))
    ks64, vs64 = float(np.float32(k_scale)), float(np.float32(v_scale))
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
        K = e4m3_to_f64(gather_tokens(k_cache, bt[s], L)) * ks64     # [L, Hkv, D]
        V = e4m3_to_f64(gather_tokens(v_cache, bt[s], L)) * vs64
        for r in my_rows:
            p = row_position(L, q_len, r - a)
            qr = bf16_bits_to_f64(q[r])
            for h in range(Hkv):
                heads = [g for g in range(Hq) if kv_head_of(g, group) == h]
                out[r, heads] = softmax_attend(qr[heads], K[:p + 1, h], V[:p + 1, h], scale64)
    return out
