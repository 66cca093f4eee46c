"""fp64 CPU oracle for the fused attention forward pass (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  It shares no code with the HIP library.
"""

from .attention import (  # noqa: F401
    NEG_INF,
    attention_backward_ref,
    attention_flops,
    attention_ref,
    fp8_e4m3_value,
    gather_pages,
    decode_fp8_ref,
    decode_paged_ref,
    decode_ref,
    decode_split_ref,
    merge_ref,
    online_softmax_ref,
    visible_keys,
)
