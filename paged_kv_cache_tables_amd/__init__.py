"""Paged GQA attention over block tables for AMD Instinct MI355X (gfx950).

The work is done by the HIP library ``libpagedkv.so`` (C ABI in
``include/pagedkv.h``); this package is a thin ctypes binding with the same
calls (the three of the bf16 cache, the append and attention of the 8-bit
E4M3 cache, the block copy of copy-on-write, the metadata check) and the host block allocator
with its radix prefix cache, taking torch tensors for device memory and
streams.  Importing
the package does not load the library; the first call does, and fails loudly
if it is missing (build it with ``python -m paged_kv_cache_tables_amd.build``).
"""
from ._lib import (  # noqa: F401
    META_FLAGS,
    NOALLOC_SCRATCH_BYTES,
    AllocatorFull,
    BlockAllocator,
    PagedKVError,
    PreparedCall,
    check_metadata,
    kv_copy_blocks,
    kv_append,
    kv_append_fp8,
    kv_bytes_per_token,
    library_path,
    load_library,
    paged_attention,
    paged_attention_append,
    paged_attention_append_noalloc,
    paged_attention_fp8,
    peak_mfma_bf16,
    peak_read,
    workspace_bytes,
)
