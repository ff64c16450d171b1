"""CPU oracle for paged GQA attention over block tables.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  The HIP library and its Python
binding never import it, and it imports nothing from them: the two share no
code, headers, tables or helpers.  The only module both sides consume is the
seeded input generator (``workloads.py``), which holds none of the method's
arithmetic.

Everything here is plain, slow and meant to be checked by eye against the
pages it cites: the byte formula, the append as a bit copy, and softmax
attention written as its definition in float64, walking the block table; for
an FP8 cache, the E4M3 code table, nearest-even quantisation with a per-pool
scale, and the same attention over the dequantised values.

Pins (tests/test_oracle_*.py) tie each function to something other than
itself: the byte counts the pages print, brute-force scalar attention on
tiny inputs, a library attention routine on dense inputs, closed forms
(length-1 context, zero query, identical keys) and invariants (placement and
block size, GQA as repeated-KV MHA, prefix sharing, poisoned tails).
"""
from .paged import (  # noqa: F401
    bf16_bits_to_f64,
    kv_bytes_per_token,
    kv_append,
    gather_tokens,
    paged_attention,
)
from .fp8 import (  # noqa: F401
    e4m3_value,
    e4m3_to_f64,
    f64_to_e4m3,
    quantize_bf16,
    kv_append_fp8,
    paged_attention_fp8,
)
