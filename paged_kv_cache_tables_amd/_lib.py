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
          -4: "HIP launch error", -5: "no free blocks",
          -6: "shape needs more than the static scratch"}

# bytes of the static device scratch behind paged_attention_append_noalloc (PKV_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


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
    lib.paged_attention_append.restype = c_int
    lib.paged_attention_append.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_void_p, c_void_p, c_int32, c_int64, c_int32, c_int32,
                                           c_int32, c_int32, c_int32, c_int64, c_int32, c_float, c_void_p,
                                           c_size_p, c_void_p]
    lib.paged_attention_append_noalloc.restype = c_int
    lib.paged_attention_append_noalloc.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                                   c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int64,
                                                   c_int32, c_int32, c_int32, c_int32, c_int32, c_int64, c_int32,
                                                   c_float, c_void_p]
    lib.kv_append_fp8.restype = c_int
    lib.kv_append_fp8.argtypes = [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_int64,
                                  c_int32, c_int32, c_int32, c_float, c_float, c_void_p]
    lib.paged_attention_fp8.restype = c_int
    lib.paged_attention_fp8.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_int32, c_int64, c_int32, c_int32, c_int32, c_int32,
                                        c_int32, c_int64, c_int32, c_float, c_float, c_float, c_void_p,
                                        c_size_p, c_void_p]
    lib.kv_copy_blocks.restype = c_int
    lib.kv_copy_blocks.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int64, c_int32, c_int32,
                                   c_int32, c_int32, c_void_p]
    i32p, i64p = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    lib.pkv_allocator_create.restype = c_void_p
    lib.pkv_allocator_create.argtypes = [c_int32, c_int32]
    lib.pkv_allocator_destroy.restype = None
    lib.pkv_allocator_destroy.argtypes = [c_void_p]
    lib.pkv_allocator_allocate.restype = c_int
    lib.pkv_allocator_allocate.argtypes = [c_void_p, i32p, c_int32, c_int32, i64p, i32p, c_int32, i32p, i32p]
    lib.pkv_allocator_free.restype = c_int
    lib.pkv_allocator_free.argtypes = [c_void_p, c_int64, i32p, c_int32]
    lib.pkv_allocator_fork.restype = c_int
    lib.pkv_allocator_fork.argtypes = [c_void_p, c_int64, c_int32, i64p, i32p, c_int32, i32p]
    lib.pkv_allocator_extend.restype = c_int
    lib.pkv_allocator_extend.argtypes = [c_void_p, c_int64, c_int32, i32p, c_int32, i32p]
    lib.pkv_allocator_prepare_write.restype = c_int
    lib.pkv_allocator_prepare_write.argtypes = [c_void_p, c_int64, c_int32, i32p, i32p]
    lib.pkv_allocator_slots.restype = c_int
    lib.pkv_allocator_slots.argtypes = [c_void_p, c_int64, c_int32, c_int32, i64p]
    lib.pkv_allocator_table.restype = c_int
    lib.pkv_allocator_table.argtypes = [c_void_p, c_int64, i32p, c_int32, i32p]
    lib.pkv_allocator_num_free.restype = c_int32
    lib.pkv_allocator_num_free.argtypes = [c_void_p]
    lib.pkv_allocator_num_cached.restype = c_int32
    lib.pkv_allocator_num_cached.argtypes = [c_void_p]
    lib.pkv_peak_read.restype = c_int
    lib.pkv_peak_read.argtypes = [c_void_p, c_int64, c_void_p, c_void_p]
    lib.pkv_peak_mfma_bf16.restype = c_int
    lib.pkv_peak_mfma_bf16.argtypes = [c_int64, c_void_p, i64p, c_void_p]
    lib.pkv_check_metadata.restype = c_int
    lib.pkv_check_metadata.argtypes = [c_void_p, c_void_p, c_void_p, c_int32, c_int64, c_int32, c_int32,
                                       c_void_p, c_int64, c_int32, c_void_p, c_void_p]
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


def peak_read(buf, sink, stream=None, prepare=False):
    """Measurement helper: one streaming read of the whole uint8 device tensor ``buf`` (size a
    multiple of 16); ``sink`` a small int32 device tensor that is never written in practice."""
    import torch
    _check(buf, "buf", torch.uint8, 1, None)
    _check(sink, "sink", torch.int32, 1, buf.device)
    lib = load_library()
    return _issue("pkv_peak_read", lib.pkv_peak_read,
                  [buf.data_ptr(), buf.numel(), sink.data_ptr(), _stream_ptr(stream, buf.device)], prepare,
                  (buf, sink))


def peak_mfma_bf16(iterations: int, sink, stream=None):
    """Measurement helper: a launch of back-to-back bf16 matrix-core products; returns its flops."""
    import torch
    _check(sink, "sink", torch.int32, 1, None)
    flops = ctypes.c_int64(0)
    lib = load_library()
    _issue("pkv_peak_mfma_bf16", lib.pkv_peak_mfma_bf16,
           [int(iterations), sink.data_ptr(), ctypes.byref(flops), _stream_ptr(stream, sink.device)], False)
    return int(flops.value)


_CARG = type(ctypes.byref(ctypes.c_int()))


class PreparedCall:
    """One library call whose tensors were checked and marshalled once: calling it issues the
    same C call again (same tensors, same stream; their contents may have changed).  For
    tight loops, where re-checking a dozen tensors per step costs more host time than the
    kernels take on the device.  Holds references to its tensors."""

    def __init__(self, name, fn, args, keep):
        self.name = name
        self._fn = fn
        self._args = [a if a is None or isinstance(a, (ctypes._SimpleCData, _CARG)) else t(a)
                      for t, a in zip(fn.argtypes, args)]
        self._keep = keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != 0:
            raise PagedKVError(self.name, st)


def _issue(name, fn, args, prepare, keep=()):
    """Make the C call now, or (prepare=True) return it as a PreparedCall."""
    if prepare:
        return PreparedCall(name, fn, args, keep)
    st = fn(*args)
    if st != 0:
        raise PagedKVError(name, st)
    return None


def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, stream=None, prepare=False):
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
    lib = load_library()
    return _issue("kv_append", lib.kv_append,
                  [k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(), T, k_cache.data_ptr(),
                   v_cache.data_ptr(), NB, bs, Hkv, D, _stream_ptr(stream, dev)],
                  prepare, (k_new, v_new, slot_mapping, k_cache, v_cache))


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


def _attention_shapes(name, out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, pool_dtype):
    """Check the tensors every attention call takes; return (NB, bs, Hkv, D, T, Hq, S, max_blocks, dev)."""
    import torch
    dev = k_cache.device
    _check(out, "out", torch.bfloat16, 3, dev)
    _check(q, "q", torch.bfloat16, 3, dev)
    if pool_dtype is None:                       # 8-bit pools
        k_cache = _check_codes(k_cache, "k_cache", 4, dev)
        v_cache = _check_codes(v_cache, "v_cache", 4, dev)
    else:
        for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
            _check(t, n, pool_dtype, 4, dev)
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
    return NB, bs, Hkv, D, T, Hq, S, block_tables.shape[1], dev


def _workspace(name, need, workspace, dev, stream=None):
    """The caller's workspace (checked), or a fresh one.  A fresh workspace comes from torch's
    caching allocator on the current stream; when the call runs on another stream it is
    recorded on that stream too, so that its memory is not handed out again before the
    kernels that use it there have finished."""
    import torch
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        if stream is not None and stream != torch.cuda.current_stream(dev):
            workspace.record_stream(stream)
    else:
        _check(workspace, "workspace", torch.uint8, 1, dev)
    return workspace


def paged_attention(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, scale: float,
                    max_query_len: int, workspace=None, stream=None, prepare=False):
    """Causal GQA attention of mixed decode/prefill rows over the paged cache, written into ``out``.

    out, q: bf16 [T, Hq, D]; pools bf16 [NB, bs, Hkv, D]; block_tables int32 [S, max_blocks];
    seq_lens int32 [S]; query_start_loc int32 [S+1]; max_query_len: host bound on rows per
    sequence.  ``workspace``: a device uint8 tensor of at least ``workspace_bytes(...)``
    bytes (allocated here if None; it needs no initialisation).  ``prepare=True`` returns
    the checked call as a PreparedCall instead of making it.
    """
    import torch
    NB, bs, Hkv, D, T, Hq, S, max_blocks, dev = _attention_shapes(
        "paged_attention", out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, torch.bfloat16)
    lib = load_library()
    need = ctypes.c_size_t(0)
    st = lib.paged_attention(None, None, None, None, None, None, None, S, T, max_blocks, max_query_len,
                             Hq, Hkv, D, NB, bs, float(scale), None, ctypes.byref(need), None)
    if st != 0:
        raise PagedKVError("paged_attention", st)
    workspace = _workspace("paged_attention", need.value, workspace, dev, stream)
    have = ctypes.c_size_t(workspace.numel())
    return _issue("paged_attention", lib.paged_attention,
                  [out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                   seq_lens.data_ptr(), query_start_loc.data_ptr(), S, T, max_blocks, max_query_len, Hq, Hkv, D,
                   NB, bs, float(scale), workspace.data_ptr(), ctypes.byref(have), _stream_ptr(stream, dev)],
                  prepare, (out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, workspace, have))


def paged_attention_append(out, q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables, seq_lens,
                           query_start_loc, scale: float, max_query_len: int, workspace=None, stream=None,
                           prepare=False):
    """kv_append then paged_attention in one call: row i of k_new / v_new (bf16 [T, Hkv, D]) is the new
    token of query row i and slot_mapping[i] (int64 [T]) its slot under block_tables.  Same result as
    the two calls; the workspace is sized as for paged_attention (``workspace_bytes``)."""
    import torch
    NB, bs, Hkv, D, T, Hq, S, max_blocks, dev = _attention_shapes(
        "paged_attention_append", out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
        torch.bfloat16)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _check(t, n, torch.bfloat16, 3, dev)
    _check(slot_mapping, "slot_mapping", torch.int64, 1, dev)
    if k_new.shape != (T, Hkv, D) or v_new.shape != (T, Hkv, D) or slot_mapping.shape[0] != T:
        raise ValueError("k_new/v_new/slot_mapping must have one row per query row")
    lib = load_library()
    need = ctypes.c_size_t(0)
    st = lib.paged_attention(None, None, None, None, None, None, None, S, T, max_blocks, max_query_len,
                             Hq, Hkv, D, NB, bs, float(scale), None, ctypes.byref(need), None)
    if st != 0:
        raise PagedKVError("paged_attention_append", st)
    workspace = _workspace("paged_attention_append", need.value, workspace, dev, stream)
    have = ctypes.c_size_t(workspace.numel())
    return _issue("paged_attention_append", lib.paged_attention_append,
                  [out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(),
                   k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), seq_lens.data_ptr(),
                   query_start_loc.data_ptr(), S, T, max_blocks, max_query_len, Hq, Hkv, D, NB, bs, float(scale),
                   workspace.data_ptr(), ctypes.byref(have), _stream_ptr(stream, dev)],
                  prepare, (out, q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables, seq_lens,
                            query_start_loc, workspace, have))


def paged_attention_append_noalloc(out, q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                                   seq_lens, query_start_loc, scale: float, max_query_len: int, stream=None,
                                   prepare=False):
    """paged_attention_append with no workspace: the library's static per-GPU scratch
    (NOALLOC_SCRATCH_BYTES) holds the partials, so neither the library nor this binding allocates
    device memory.  Raises PagedKVError (status -6) for shapes that need more scratch than that.
    Calls that may overlap on one GPU share the scratch and race: order them."""
    import torch
    NB, bs, Hkv, D, T, Hq, S, max_blocks, dev = _attention_shapes(
        "paged_attention_append_noalloc", out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
        torch.bfloat16)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _check(t, n, torch.bfloat16, 3, dev)
    _check(slot_mapping, "slot_mapping", torch.int64, 1, dev)
    if k_new.shape != (T, Hkv, D) or v_new.shape != (T, Hkv, D) or slot_mapping.shape[0] != T:
        raise ValueError("k_new/v_new/slot_mapping must have one row per query row")
    lib = load_library()
    return _issue("paged_attention_append_noalloc", lib.paged_attention_append_noalloc,
                  [out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(),
                   k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), seq_lens.data_ptr(),
                   query_start_loc.data_ptr(), S, T, max_blocks, max_query_len, Hq, Hkv, D, NB, bs, float(scale),
                   _stream_ptr(stream, dev)],
                  prepare, (out, q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables, seq_lens,
                            query_start_loc))


def _check_codes(t, name, ndim, device):
    """An 8-bit pool: uint8 (or torch.float8_e4m3fn) device tensor."""
    import torch
    if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    _check(t, name, torch.uint8, ndim, device)
    return t


def kv_append_fp8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale: float, v_scale: float,
                  stream=None, prepare=False):
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
    lib = load_library()
    return _issue("kv_append_fp8", lib.kv_append_fp8,
                  [k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(), T, k_cache.data_ptr(),
                   v_cache.data_ptr(), NB, bs, Hkv, D, float(k_scale), float(v_scale), _stream_ptr(stream, dev)],
                  prepare, (k_new, v_new, slot_mapping, k_cache, v_cache))


def paged_attention_fp8(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, scale: float,
                        max_query_len: int, k_scale: float, v_scale: float, workspace=None,
                        stream=None, prepare=False):
    """paged_attention over E4M3 pools (uint8 [NB, bs, Hkv, D]) with per-pool scales k_scale, v_scale.
    The workspace is sized as for paged_attention (``workspace_bytes``)."""
    NB, bs, Hkv, D, T, Hq, S, max_blocks, dev = _attention_shapes(
        "paged_attention_fp8", out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, None)
    import torch
    if k_cache.dtype == torch.float8_e4m3fn:
        k_cache, v_cache = k_cache.view(torch.uint8), v_cache.view(torch.uint8)
    lib = load_library()
    need = ctypes.c_size_t(0)
    st = lib.paged_attention_fp8(None, None, None, None, None, None, None, S, T, max_blocks, max_query_len,
                                 Hq, Hkv, D, NB, bs, float(scale), float(k_scale), float(v_scale), None,
                                 ctypes.byref(need), None)
    if st != 0:
        raise PagedKVError("paged_attention_fp8", st)
    workspace = _workspace("paged_attention_fp8", need.value, workspace, dev, stream)
    have = ctypes.c_size_t(workspace.numel())
    return _issue("paged_attention_fp8", lib.paged_attention_fp8,
                  [out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                   seq_lens.data_ptr(), query_start_loc.data_ptr(), S, T, max_blocks, max_query_len, Hq, Hkv, D,
                   NB, bs, float(scale), float(k_scale), float(v_scale), workspace.data_ptr(), ctypes.byref(have),
                   _stream_ptr(stream, dev)],
                  prepare, (out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, workspace, have))


def kv_copy_blocks(k_cache, v_cache, src, dst, stream=None) -> None:
    """Copy whole blocks src[i] -> dst[i] (int32 device tensors) in both pools (bf16 or uint8)."""
    import torch
    dev = k_cache.device
    if k_cache.dtype == torch.float8_e4m3fn:
        k_cache, v_cache = k_cache.view(torch.uint8), v_cache.view(torch.uint8)
    if k_cache.dtype not in (torch.bfloat16, torch.uint8) or v_cache.dtype != k_cache.dtype:
        raise TypeError("pools must both be bf16 or both uint8")
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _check(t, n, k_cache.dtype, 4, dev)
    for t, n in ((src, "src"), (dst, "dst")):
        _check(t, n, torch.int32, 1, dev)
    if src.shape != dst.shape or v_cache.shape != k_cache.shape:
        raise ValueError("src/dst or pool shapes differ")
    NB, bs, Hkv, D = k_cache.shape
    st = load_library().kv_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), src.data_ptr(), dst.data_ptr(),
                                       src.shape[0], NB, bs, Hkv, D, k_cache.element_size(),
                                       _stream_ptr(stream, dev))
    if st != 0:
        raise PagedKVError("kv_copy_blocks", st)


# Flags of pkv_check_metadata (include/pagedkv.h), by bit.
META_FLAGS = {
    0x01: "query_start_loc: [0] != 0, decreasing, or last != num_q_tokens",
    0x02: "a sequence has more rows than max_query_len",
    0x04: "a length is negative, or smaller than its sequence's rows",
    0x08: "a length exceeds max_blocks_per_seq * block_size",
    0x10: "a needed block-table entry lies outside the pool",
    0x20: "a slot lies outside the pool",
    0x40: "a row's slot is not its position's slot under the block table",
}


def check_metadata(block_tables, seq_lens, query_start_loc, num_q_tokens, max_query_len, num_blocks,
                   block_size, slot_mapping=None, error_word=None, stream=None):
    """Device check of one step's metadata against the contract of kv_append and
    paged_attention (pkv_check_metadata).  With ``error_word`` (an int32 device tensor of one
    element) the check is only enqueued and None is returned; without it a one-element tensor
    is allocated here, the stream synchronised and the flags returned (0: the contract holds;
    see META_FLAGS)."""
    import torch
    dev = block_tables.device
    _check(block_tables, "block_tables", torch.int32, 2, dev)
    _check(seq_lens, "seq_lens", torch.int32, 1, dev)
    _check(query_start_loc, "query_start_loc", torch.int32, 1, dev)
    S, max_blocks = block_tables.shape
    if seq_lens.shape[0] != S or query_start_loc.shape[0] != S + 1:
        raise ValueError("block_tables, seq_lens and query_start_loc disagree on the number of sequences")
    slots_ptr = None
    if slot_mapping is not None:
        _check(slot_mapping, "slot_mapping", torch.int64, 1, dev)
        if slot_mapping.shape[0] != num_q_tokens:
            raise ValueError("slot_mapping must have num_q_tokens entries")
        slots_ptr = slot_mapping.data_ptr()
    own = error_word is None
    if own:
        error_word = torch.empty(1, dtype=torch.int32, device=dev)
    _check(error_word, "error_word", torch.int32, 1, dev)
    st = load_library().pkv_check_metadata(block_tables.data_ptr(), seq_lens.data_ptr(),
                                           query_start_loc.data_ptr(), S, int(num_q_tokens), max_blocks,
                                           int(max_query_len), slots_ptr, int(num_blocks), int(block_size),
                                           error_word.data_ptr(), _stream_ptr(stream, dev))
    if st != 0:
        raise PagedKVError("pkv_check_metadata", st)
    if not own:
        return None
    (torch.cuda.current_stream(dev) if stream is None else stream).synchronize()
    return int(error_word.item())


class AllocatorFull(RuntimeError):
    """No free blocks for the request, even after evicting every unreferenced cached prefix."""


class BlockAllocator:
    """The library's host block allocator with a radix prefix cache (pkv_allocator_*).

    allocate(tokens, n_total) -> (id, blocks, cached prefix length); free(id, tokens);
    fork(id, n_tokens) -> (id, blocks); extend(id, n_total) -> blocks;
    prepare_write(id, pos) -> None or (src, dst); slots(id, start, count); table(id).
    ``error``: the exception class raised when blocks run out (default AllocatorFull)."""

    def __init__(self, num_blocks: int, block_size: int, error=AllocatorFull):
        self._lib = load_library()
        h = self._lib.pkv_allocator_create(int(num_blocks), int(block_size))
        if not h:
            raise ValueError("num_blocks >= 2 and block_size >= 1 are required")
        self._h = ctypes.c_void_p(h)
        self.num_blocks, self.block_size, self._error = int(num_blocks), int(block_size), error
        self._cap = {}

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and self._lib is not None:
            self._lib.pkv_allocator_destroy(h)
            self._h = None

    def _status(self, st, what, key=None):
        if st == -5:
            raise self._error(f"{what}: no free blocks")
        if st != 0:
            if key is not None and key not in self._cap:
                raise KeyError(key)
            raise ValueError(f"{what}: {STATUS.get(st, st)}")

    @staticmethod
    def _i32(seq):
        """int32 token ids as a C pointer (a contiguous int32 numpy array is passed as is)."""
        import numpy as np
        arr = np.ascontiguousarray(seq, dtype=np.int32)
        if arr.size == 0:
            arr = np.zeros(1, dtype=np.int32)
        return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))

    def allocate(self, tokens, n_total: int):
        keep, toks = self._i32(tokens)
        cap = max(1, -(-int(n_total) // self.block_size))
        out = (ctypes.c_int32 * cap)()
        aid, nb, pre = ctypes.c_int64(0), ctypes.c_int32(0), ctypes.c_int32(0)
        st = self._lib.pkv_allocator_allocate(self._h, toks, len(tokens), int(n_total), ctypes.byref(aid), out, cap,
                                              ctypes.byref(nb), ctypes.byref(pre))
        self._status(st, "allocate")
        self._cap[aid.value] = nb.value
        return aid.value, list(out[:nb.value]), pre.value

    def free(self, alloc_id: int, tokens) -> None:
        keep, toks = self._i32(tokens)
        st = self._lib.pkv_allocator_free(self._h, int(alloc_id), toks, len(tokens))
        self._status(st, "free", alloc_id)
        del self._cap[alloc_id]

    def table(self, alloc_id: int):
        n = ctypes.c_int32(0)
        st = self._lib.pkv_allocator_table(self._h, int(alloc_id), None, 0, ctypes.byref(n))
        self._status(st, "table", alloc_id)
        out = (ctypes.c_int32 * max(1, n.value))()
        st = self._lib.pkv_allocator_table(self._h, int(alloc_id), out, n.value, ctypes.byref(n))
        self._status(st, "table", alloc_id)
        return list(out[:n.value])

    def fork(self, alloc_id: int, n_tokens: int):
        if alloc_id not in self._cap:
            raise KeyError(alloc_id)
        cap = max(1, self._cap[alloc_id])
        out = (ctypes.c_int32 * cap)()
        nid, nb = ctypes.c_int64(0), ctypes.c_int32(0)
        st = self._lib.pkv_allocator_fork(self._h, int(alloc_id), int(n_tokens), ctypes.byref(nid), out, cap,
                                          ctypes.byref(nb))
        self._status(st, "fork", alloc_id)
        self._cap[nid.value] = nb.value
        return nid.value, list(out[:nb.value])

    def extend(self, alloc_id: int, n_total: int):
        if alloc_id not in self._cap:
            raise KeyError(alloc_id)
        cap = max(self._cap[alloc_id], -(-int(n_total) // self.block_size), 1)
        out = (ctypes.c_int32 * cap)()
        nb = ctypes.c_int32(0)
        st = self._lib.pkv_allocator_extend(self._h, int(alloc_id), int(n_total), out, cap, ctypes.byref(nb))
        self._status(st, "extend", alloc_id)
        self._cap[alloc_id] = nb.value
        return list(out[:nb.value])

    def prepare_write(self, alloc_id: int, pos: int):
        src, dst = ctypes.c_int32(-1), ctypes.c_int32(-1)
        st = self._lib.pkv_allocator_prepare_write(self._h, int(alloc_id), int(pos), ctypes.byref(src),
                                                   ctypes.byref(dst))
        self._status(st, "prepare_write", alloc_id)
        return None if src.value < 0 else (src.value, dst.value)

    def slots(self, alloc_id: int, start: int, count: int):
        out = (ctypes.c_int64 * max(1, int(count)))()
        st = self._lib.pkv_allocator_slots(self._h, int(alloc_id), int(start), int(count), out)
        self._status(st, "slots", alloc_id)
        return list(out[:int(count)])

    def num_free(self) -> int:
        return int(self._lib.pkv_allocator_num_free(self._h))

    def num_cached(self) -> int:
        return int(self._lib.pkv_allocator_num_cached(self._h))
