"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, computes the byte formula, and rejects bad arguments on the host
before any HIP call (each case below fails validation, so no kernel runs)."""
import ctypes
import json
import os
import re
import subprocess

import pytest

import paged_kv_cache_tables_amd as pkv
from paged_kv_cache_tables_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EWORKSPACE, PKV_ESCRATCH = 0, -1, -2, -3, -6


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkv.library_path()):
        pytest.fail("libpagedkv.so is not built (python -m paged_kv_cache_tables_amd.build)")
    return pkv.load_library()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"PKV_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("kv_append", "paged_attention", "kv_bytes_per_token"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", pkv.library_path()], capture_output=True, text=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def test_kv_bytes_per_token_golden(lib, golden_dir):
    g = json.load(open(os.path.join(golden_dir, "kv_bytes_per_token.json")))
    for case in g["per_token"]:
        assert lib.kv_bytes_per_token(*case["args"]) == case["expected"], case["cite"]
    for bad in [(0, 8, 128, 2), (80, -8, 128, 2), (80, 8, 0, 2), (80, 8, 128, -1), (2 ** 62, 8, 128, 2)]:
        assert lib.kv_bytes_per_token(*bad) == -1


FAKE = 0x10000   # aligned, never dereferenced: every call below fails validation first


def append_args(**over):
    a = dict(k_new=FAKE, v_new=FAKE, slot_mapping=FAKE, num_tokens=4, k_cache=FAKE, v_cache=FAKE,
             num_blocks=8, block_size=16, num_kv_heads=2, head_dim=64, stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("over,expect", [
    (dict(k_new=None), PKV_EINVAL),
    (dict(slot_mapping=None), PKV_EINVAL),
    (dict(num_tokens=-1), PKV_EINVAL),
    (dict(num_blocks=0), PKV_EINVAL),
    (dict(block_size=0), PKV_EINVAL),
    (dict(head_dim=60), PKV_EUNSUPPORTED),
    (dict(k_cache=FAKE + 8), PKV_EINVAL),          # not 16-byte aligned
    (dict(num_tokens=0), PKV_OK),                   # nothing to do, nothing launched
    (dict(num_tokens=0, k_new=None, slot_mapping=None), PKV_OK),   # empty tensors have null data
])
def test_kv_append_validation(lib, over, expect):
    assert lib.kv_append(*append_args(**over)) == expect


def attn_args(**over):
    n = ctypes.c_size_t(1 << 30)
    a = dict(out=FAKE, q=FAKE, k_cache=FAKE, v_cache=FAKE, block_tables=FAKE, seq_lens=FAKE,
             qsl=FAKE, num_seqs=4, num_q_tokens=8, max_blocks=4, max_query_len=5, Hq=4, Hkv=2, D=64,
             num_blocks=64, bs=16, scale=0.125, workspace=None, workspace_bytes=ctypes.byref(n),
             stream=None)
    a.update(over)
    return list(a.values())


def test_workspace_query_and_size(lib):
    n = ctypes.c_size_t(0)
    assert lib.paged_attention(*attn_args(workspace_bytes=ctypes.byref(n))) == PKV_OK
    # decode partials: 2 slots of 16 columns of (64 + 2) floats per decode wave (2048 waves on a
    # 256-CU device, also the figure without a device), each array 256-byte aligned
    assert n.value >= 2048 * 2 * 16 * 66 * 4
    small = ctypes.c_size_t(n.value - 1)
    assert lib.paged_attention(*attn_args(workspace=FAKE, workspace_bytes=ctypes.byref(small))) == PKV_EWORKSPACE
    assert pkv.workspace_bytes(4, 4, 2, 64, 4, 16, max_query_len=5) == n.value
    # the partials do not depend on the batch: only the piece records and the prefill work
    # list grow with the sequences and their length
    assert pkv.workspace_bytes(4, 4, 2, 64, 4, 16, max_query_len=1) == n.value
    assert pkv.workspace_bytes(4, 4, 2, 64, 4, 16, max_query_len=500) == n.value
    assert pkv.workspace_bytes(400, 4, 2, 64, 4, 16) > n.value
    assert pkv.workspace_bytes(4, 4, 2, 64, 4000, 16) > n.value
    # D 128: 34 MB of partials for any batch; every task configuration fits the static scratch
    assert pkv.workspace_bytes(256, 64, 8, 128, 512, 16) < pkv.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("over,expect", [
    (dict(workspace_bytes=None), PKV_EINVAL),
    (dict(Hq=6, Hkv=4), PKV_EINVAL),               # not a multiple
    (dict(Hq=32, Hkv=1), PKV_EUNSUPPORTED),        # group of 32 not built
    (dict(D=96), PKV_EUNSUPPORTED),
    (dict(bs=12), PKV_EUNSUPPORTED),
    (dict(num_seqs=-1), PKV_EINVAL),
    (dict(max_blocks=0), PKV_EINVAL),
    (dict(scale=float("nan")), PKV_EINVAL),
    (dict(num_blocks=0), PKV_EINVAL),
])
def test_paged_attention_validation(lib, over, expect):
    assert lib.paged_attention(*attn_args(**over)) == expect


def test_paged_attention_checks_pointers_before_launch(lib):
    n = ctypes.c_size_t(1 << 30)
    for field in ("out", "q", "k_cache", "v_cache", "block_tables", "seq_lens", "qsl"):
        args = attn_args(workspace=FAKE, workspace_bytes=ctypes.byref(n), **{field: None})
        assert lib.paged_attention(*args) == PKV_EINVAL, field
    args = attn_args(workspace=FAKE + 16, workspace_bytes=ctypes.byref(n))
    assert lib.paged_attention(*args) == PKV_EINVAL                     # workspace alignment
    args = attn_args(workspace=FAKE, workspace_bytes=ctypes.byref(n), max_query_len=0)
    assert lib.paged_attention(*args) == PKV_EINVAL                     # rows but no bound
    args = attn_args(workspace=FAKE, workspace_bytes=ctypes.byref(n), num_q_tokens=0)
    assert lib.paged_attention(*args) == PKV_OK                         # empty batch: no launch


def test_noalloc_rejects_before_any_device_call(lib):
    """paged_attention_append_noalloc checks its arguments and the scratch its shape needs on the
    host: invalid shapes and shapes beyond the static scratch return before any HIP call."""
    def call(**over):
        a = dict(num_seqs=256, T=256, max_blocks=512, max_query_len=1, Hq=64, Hkv=8, D=128, NB=1 << 16,
                 bs=16, scale=0.088)
        a.update(over)
        return lib.paged_attention_append_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                  a["num_seqs"], a["T"], a["max_blocks"], a["max_query_len"],
                                                  a["Hq"], a["Hkv"], a["D"], a["NB"], a["bs"], a["scale"], None)
    # 4096 sequences of up to 131072 tokens: the prefill work list alone exceeds the scratch
    need = pkv.workspace_bytes(4096, 64, 8, 128, 8192, 16, 1)
    assert need > pkv.NOALLOC_SCRATCH_BYTES
    assert call(num_seqs=4096, T=4096, max_blocks=8192) == PKV_ESCRATCH
    assert call(Hq=6, Hkv=4) == PKV_EINVAL
    assert call(D=96) == PKV_EUNSUPPORTED
    assert call(scale=float("inf")) == PKV_EINVAL
    assert pkv.workspace_bytes(64, 32, 8, 128, 256, 16, 1) <= pkv.NOALLOC_SCRATCH_BYTES


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert lib.pkv_status_string(code).decode() == _lib.STATUS[code]


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "PKG", str(tmp_path))
    with pytest.raises(FileNotFoundError):
        _lib.kv_bytes_per_token(1, 1, 1, 1)


# -- 8-bit cache ---------------------------------------------------------------

def append_fp8_args(**over):
    a = dict(k_new=FAKE, v_new=FAKE, slot_mapping=FAKE, num_tokens=4, k_cache=FAKE, v_cache=FAKE,
             num_blocks=8, block_size=16, num_kv_heads=2, head_dim=64, k_scale=0.5, v_scale=0.25, stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("over,expect", [
    (dict(k_new=None), PKV_EINVAL),
    (dict(num_tokens=-1), PKV_EINVAL),
    (dict(k_scale=0.0), PKV_EINVAL),
    (dict(v_scale=-1.0), PKV_EINVAL),
    (dict(k_scale=float("inf")), PKV_EINVAL),
    (dict(v_scale=float("nan")), PKV_EINVAL),
    (dict(head_dim=72), PKV_EUNSUPPORTED),          # rows of codes move in 16-byte chunks
    (dict(v_cache=FAKE + 8), PKV_EINVAL),
    (dict(num_tokens=0, k_new=None, slot_mapping=None), PKV_OK),
])
def test_kv_append_fp8_validation(lib, over, expect):
    assert lib.kv_append_fp8(*append_fp8_args(**over)) == expect


def attn_fp8_args(**over):
    n = ctypes.c_size_t(1 << 30)
    a = dict(out=FAKE, q=FAKE, k_cache=FAKE, v_cache=FAKE, block_tables=FAKE, seq_lens=FAKE,
             qsl=FAKE, num_seqs=4, num_q_tokens=8, max_blocks=4, max_query_len=5, Hq=4, Hkv=2, D=64,
             num_blocks=64, bs=16, scale=0.125, k_scale=0.5, v_scale=0.25, workspace=None,
             workspace_bytes=ctypes.byref(n), stream=None)
    a.update(over)
    return list(a.values())


def test_fp8_workspace_matches_bf16(lib):
    for shape in (dict(), dict(D=128, Hq=32, Hkv=8, max_query_len=1), dict(bs=32, max_query_len=300)):
        a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
        assert lib.paged_attention_fp8(*attn_fp8_args(workspace_bytes=ctypes.byref(a), **shape)) == PKV_OK
        assert lib.paged_attention(*attn_args(workspace_bytes=ctypes.byref(b), **shape)) == PKV_OK
        assert a.value == b.value > 0


@pytest.mark.parametrize("over,expect", [
    (dict(k_scale=0.0), PKV_EINVAL),
    (dict(v_scale=float("nan")), PKV_EINVAL),
    (dict(k_scale=-2.0), PKV_EINVAL),
    (dict(bs=8), PKV_EUNSUPPORTED),                 # d 64 codes: a wave-wide load spans 16 slots
    (dict(D=96), PKV_EUNSUPPORTED),
    (dict(Hq=6, Hkv=4), PKV_EINVAL),
    (dict(scale=float("inf")), PKV_EINVAL),
])
def test_paged_attention_fp8_validation(lib, over, expect):
    assert lib.paged_attention_fp8(*attn_fp8_args(**over)) == expect


def test_paged_attention_fp8_accepts_d128_bs8(lib):
    n = ctypes.c_size_t(0)
    assert lib.paged_attention_fp8(*attn_fp8_args(D=128, bs=8, workspace_bytes=ctypes.byref(n))) == PKV_OK


def test_paged_attention_fp8_checks_pointers_before_launch(lib):
    n = ctypes.c_size_t(1 << 30)
    for field in ("out", "q", "k_cache", "v_cache", "block_tables", "seq_lens", "qsl"):
        args = attn_fp8_args(workspace=FAKE, workspace_bytes=ctypes.byref(n), **{field: None})
        assert lib.paged_attention_fp8(*args) == PKV_EINVAL, field


def attn_append_args(**over):
    n = ctypes.c_size_t(1 << 30)
    a = dict(out=FAKE, q=FAKE, k_new=FAKE, v_new=FAKE, slot_mapping=FAKE, k_cache=FAKE, v_cache=FAKE,
             block_tables=FAKE, seq_lens=FAKE, qsl=FAKE, num_seqs=4, num_q_tokens=8, max_blocks=4,
             max_query_len=5, Hq=4, Hkv=2, D=64, num_blocks=64, bs=16, scale=0.125, workspace=None,
             workspace_bytes=ctypes.byref(n), stream=None)
    a.update(over)
    return list(a.values())


def test_paged_attention_append_workspace_matches(lib):
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.paged_attention(*attn_args(workspace_bytes=ctypes.byref(a))) == PKV_OK
    assert lib.paged_attention_append(*attn_append_args(workspace_bytes=ctypes.byref(b))) == PKV_OK
    assert a.value == b.value


@pytest.mark.parametrize("over,expect", [
    (dict(workspace_bytes=None), PKV_EINVAL),
    (dict(Hq=6, Hkv=4), PKV_EINVAL),
    (dict(D=96), PKV_EUNSUPPORTED),
    (dict(bs=12), PKV_EUNSUPPORTED),
    (dict(scale=float("nan")), PKV_EINVAL),
])
def test_paged_attention_append_validation(lib, over, expect):
    assert lib.paged_attention_append(*attn_append_args(**over)) == expect


def test_paged_attention_append_checks_pointers_before_launch(lib):
    n = ctypes.c_size_t(1 << 30)
    for field in ("out", "q", "k_new", "v_new", "slot_mapping", "k_cache", "v_cache", "block_tables",
                  "seq_lens", "qsl"):
        args = attn_append_args(workspace=FAKE, workspace_bytes=ctypes.byref(n), **{field: None})
        assert lib.paged_attention_append(*args) == PKV_EINVAL, field
    for field, off in (("k_new", 8), ("v_new", 8), ("slot_mapping", 4)):
        args = attn_append_args(workspace=FAKE, workspace_bytes=ctypes.byref(n), **{field: FAKE + off})
        assert lib.paged_attention_append(*args) == PKV_EINVAL, field   # misaligned
    args = attn_append_args(workspace=FAKE, workspace_bytes=ctypes.byref(n), num_q_tokens=0)
    assert lib.paged_attention_append(*args) == PKV_OK                 # empty batch: no launch


def test_peak_helpers_validate_before_launch(lib):
    flops = ctypes.c_int64(0)
    assert lib.pkv_peak_read(None, 1 << 20, FAKE, None) == PKV_EINVAL
    assert lib.pkv_peak_read(FAKE, 1 << 20, None, None) == PKV_EINVAL
    assert lib.pkv_peak_read(FAKE, 1000, FAKE, None) == PKV_EINVAL          # not a multiple of 16
    assert lib.pkv_peak_read(FAKE + 8, 1 << 20, FAKE, None) == PKV_EINVAL   # misaligned
    assert lib.pkv_peak_mfma_bf16(0, FAKE, ctypes.byref(flops), None) == PKV_EINVAL
    assert lib.pkv_peak_mfma_bf16(10, None, ctypes.byref(flops), None) == PKV_EINVAL
    assert lib.pkv_peak_mfma_bf16(10, FAKE, None, None) == PKV_EINVAL


def check_args(**over):
    a = dict(bt=FAKE, sl=FAKE, qsl=FAKE, num_seqs=2, num_q_tokens=3, max_blocks=4, max_query_len=2,
             slots=None, num_blocks=8, block_size=16, error_word=FAKE, stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("over", [
    dict(error_word=None), dict(qsl=None), dict(bt=None), dict(sl=None), dict(num_seqs=-1),
    dict(num_q_tokens=-1), dict(max_query_len=-1), dict(num_blocks=-1), dict(block_size=0),
    dict(max_blocks=0),
])
def test_check_metadata_validation(lib, over):
    assert lib.pkv_check_metadata(*check_args(**over)) == PKV_EINVAL
