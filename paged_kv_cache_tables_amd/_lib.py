"""ctypes binding of libpagedkv.so: argument marshalling only.

Each function checks that tensors have the dtype, device, shape and layout the
C ABI expects, passes raw pointers and the current (or given) stream, and
raises ``PagedKVError`` on a non-zero status.  No arithmetic of the method
happens here, and there is no fallback: without the library every call raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libpagedkv.so"
_lib = None

STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported shape", -3: "workspace too small",
          -4: "HIP launch error"}


class PagedKVError(RuntimeError):
    def __init__(self, call: str, status: int):
        super().__init__(f"{call} failed: {STATUS.get(status, 'unknown')} ({status})")
        self.status = status


def library_path() -> str:
    return os.path.join(PKG, _LIB_NAME)


def load_library() -> ctypes.CDLL:
    """Load the in-tree HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m paged_kv_cache_tables_amd.build`")
    lib = ctypes.CDLL(path)
    c_void_p, c_int, c_int32, c_int64, c_float, c_size_p = (
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
        ctypes.POINTER(ctypes.c_size_t))
    lib.kv_bytes_per_token.restype = c_int64
    lib.kv_bytes_per_token.argtypes = [c_int64, c_int64, c_int64, c_int64]
    lib.kv_append.restype = c_int
    lib.kv_append.argtypes = [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_int64,
                              c_int32, c_int32, c_int32, c_void_p]
    lib.paged_attention.restype = c_int
    lib.paged_attention.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_int32, c_int64, c_int32, c_int32, c_int32, c_int32,
                                    c_int32, c_int64, c_int32, c_float, c_void_p, c_size_p, c_void_p]
    lib.kv_append_fp8.restype = c_int
    lib.kv_append_fp8.argtypes = [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_int64,
                                  c_int32, c_int32, c_int32, c_float, c_float, c_void_p]
    lib.paged_attention_fp8.restype = c_int
    lib.paged_attention_fp8.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_int32, c_int64, c_int32, c_int32, c_int32, c_int32,
                                        c_int32, c_int64, c_int32, c_float, c_float, c_float, c_void_p,
                                        c_size_p, c_void_p]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_status_string.argtypes = [c_int]
    _lib = lib
    return lib


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """2 x layers x KV heads x head_dim x bytes; -1 for invalid arguments (C ABI semantics)."""
    return int(load_library().kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dtype_bytes))


def _stream_ptr(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t, name, dtype, ndim=None, device=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """Scatter new K/V rows [T, Hkv, D] (bf16) into pools [NB, bs, Hkv, D] at slot_mapping (int64 [T])."""
    import torch
    dev = k_cache.device
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _check(t, n, torch.bfloat16, 3, dev)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _check(t, n, torch.bfloat16, 4, dev)
    _check(slot_mapping, "slot_mapping", torch.int64, 1, dev)
    NB, bs, Hkv, D = k_cache.shape
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    T = k_new.shape[0]
    if k_new.shape != (T, Hkv, D) or v_new.shape != (T, Hkv, D) or slot_mapping.shape[0] != T:
        raise ValueError("k_new/v_new/slot_mapping shapes do not match the pool")
    st = load_library().kv_append(k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(), T,
                                  k_cache.data_ptr(), v_cache.data_ptr(), NB, bs, Hkv, D,
                                  _stream_ptr(stream, dev))
    if st != 0:
        raise PagedKVError("kv_append", st)


def workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    max_blocks_per_seq: int, block_size: int, max_query_len: int = 1,
                    num_blocks: int = 1) -> int:
    """Size of the split-K workspace paged_attention needs (query mode of the C call)."""
    n = ctypes.c_size_t(0)
    st = load_library().paged_attention(None, None, None, None, None, None, None, num_seqs, 0,
                                        max_blocks_per_seq, max_query_len, num_q_heads, num_kv_heads, head_dim,
                                        num_blocks, block_size, 1.0, None, ctypes.byref(n), None)
    if st != 0:
        raise PagedKVError("paged_attention(workspace query)", st)
    return int(n.value)


def paged_attention(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, scale: float,
                    max_query_len: int, workspace=None, stream=None) -> None:
    """Causal GQA attention of mixed decode/prefill rows over the paged cache, written into ``out``.

    out, q: bf16 [T, Hq, D]; pools bf16 [NB, bs, Hkv, D]; block_tables int32 [S, max_blocks];
    seq_lens int32 [S]; query_start_loc int32 [S+1]; max_query_len: host bound on rows per
    sequence.  ``workspace``: a device uint8 tensor of at least ``workspace_bytes(...)``
    bytes (allocated here if None).
    """
    import torch
    dev = k_cache.device
    _check(out, "out", torch.bfloat16, 3, dev)
    _check(q, "q", torch.bfloat16, 3, dev)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _check(t, n, torch.bfloat16, 4, dev)
    _check(block_tables, "block_tables", torch.int32, 2, dev)
    _check(seq_lens, "seq_lens", torch.int32, 1, dev)
    _check(query_start_loc, "query_start_loc", torch.int32, 1, dev)
    NB, bs, Hkv, D = k_cache.shape
    T, Hq, Dq = q.shape
    S = seq_lens.shape[0]
    if Dq != D or out.shape != q.shape or v_cache.shape != k_cache.shape:
        raise ValueError("q/out/pool shapes do not match")
    if query_start_loc.shape[0] != S + 1 or block_tables.shape[0] != S:
        raise ValueError("query_start_loc must be [S+1] and block_tables [S, max_blocks]")
    max_blocks = block_tables.shape[1]
    lib = load_library()
    need = ctypes.c_size_t(0)
    st = lib.paged_attention(None, None, None, None, None, None, None, S, T, max_blocks, max_query_len,
                             Hq, Hkv, D, NB, bs, float(scale), None, ctypes.byref(need), None)
    if st != 0:
        raise PagedKVError("paged_attention", st)
    if workspace is None:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=dev)
    else:
        _check(workspace, "workspace", torch.uint8, 1, dev)
    have = ctypes.c_size_t(workspace.numel())
    st = lib.paged_attention(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                             block_tables.data_ptr(), seq_lens.data_ptr(), query_start_loc.data_ptr(),
                             S, T, max_blocks, max_query_len, Hq, Hkv, D, NB, bs, float(scale),
                             workspace.data_ptr(), ctypes.byref(have), _stream_ptr(stream, dev))
    if st != 0:
        raise PagedKVError("paged_attention", st)


def _check_codes(t, name, ndim, device):
    """An 8-bit pool: uint8 (or torch.float8_e4m3fn) device tensor."""
    import torch
    if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    _check(t, name, torch.uint8, ndim, device)
    return t


def kv_append_fp8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale: float, v_scale: float,
                  stream=None) -> None:
    """Quantise new K/V rows [T, Hkv, D] (bf16) into E4M3 pools [NB, bs, Hkv, D] (uint8) at slot_mapping."""
    import torch
    dev = k_cache.device
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _check(t, n, torch.bfloat16, 3, dev)
    k_cache = _check_codes(k_cache, "k_cache", 4, dev)
    v_cache = _check_codes(v_cache, "v_cache", 4, dev)
    _check(slot_mapping, "slot_mapping", torch.int64, 1, dev)
    NB, bs, Hkv, D = k_cache.shape
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    T = k_new.shape[0]
    if k_new.shape != (T, Hkv, D) or v_new.shape != (T, Hkv, D) or slot_mapping.shape[0] != T:
        raise ValueError("k_new/v_new/slot_mapping shapes do not match the pool")
    st = load_library().kv_append_fp8(k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(), T,
                                      k_cache.data_ptr(), v_cache.data_ptr(), NB, bs, Hkv, D,
                                      float(k_scale), float(v_scale), _stream_ptr(stream, dev))
    if st != 0:
        raise PagedKVError("kv_append_fp8", st)


def paged_attention_fp8(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, scale: float,
                        max_query_len: int, k_scale: float, v_scale: float, workspace=None,
                        stream=None) -> None:
    """paged_attention over E4M3 pools (uint8 [NB, bs, Hkv, D]) with per-pool scales k_scale, v_scale.
    The workspace is sized as for paged_attention (``workspace_bytes``)."""
    import torch
    dev = k_cache.device
    _check(out, "out", torch.bfloat16, 3, dev)
    _check(q, "q", torch.bfloat16, 3, dev)
    k_cache = _check_codes(k_cache, "k_cache", 4, dev)
    v_cache = _check_codes(v_cache, "v_cache", 4, dev)
    _check(block_tables, "block_tables", torch.int32, 2, dev)
    _check(seq_lens, "seq_lens", torch.int32, 1, dev)
    _check(query_start_loc, "query_start_loc", torch.int32, 1, dev)
    NB, bs, Hkv, D = k_cache.shape
    T, Hq, Dq = q.shape
    S = seq_lens.shape[0]
    if Dq != D or out.shape != q.shape or v_cache.shape != k_cache.shape:
        raise ValueError("q/out/pool shapes do not match")
    if query_start_loc.shape[0] != S + 1 or block_tables.shape[0] != S:
        raise ValueError("query_start_loc must be [S+1] and block_tables [S, max_blocks]")
    max_blocks = block_tables.shape[1]
    lib = load_library()
    need = ctypes.c_size_t(0)
    st = lib.paged_attention_fp8(None, None, None, None, None, None, None, S, T, max_blocks, max_query_len,
                                 Hq, Hkv, D, NB, bs, float(scale), float(k_scale), float(v_scale), None,
                                 ctypes.byref(need), None)
    if st != 0:
        raise PagedKVError("paged_attention_fp8", st)
    if workspace is None:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=dev)
    else:
        _check(workspace, "workspace", torch.uint8, 1, dev)
    have = ctypes.c_size_t(workspace.numel())
    st = lib.paged_attention_fp8(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                 block_tables.data_ptr(), seq_lens.data_ptr(), query_start_loc.data_ptr(),
                                 S, T, max_blocks, max_query_len, Hq, Hkv, D, NB, bs, float(scale),
                                 float(k_scale), float(v_scale), workspace.data_ptr(), ctypes.byref(have),
                                 _stream_ptr(stream, dev))
    if st != 0:
        raise PagedKVError("paged_attention_fp8", st)
