"""Fused attention forward for MI355X (gfx950): prefill, split-KV decode, LSE merge.

The computation lives in hand-written HIP kernels behind a C ABI
(``include/attn_fwd.h``, built as ``libattnfwd.so``); this package only
marshals torch device tensors into that ABI.  Importing it does not load the
library; the first call does, and raises if the library has not been built.
"""

from ._binding import (  # noqa: F401
    DECODE_WORKSPACE_HEADER,
    LIB_PATH,
    AttnError,
    backward,
    backward_workspace_size,
    combine,
    decode,
    decode_fp8,
    decode_noalloc,
    decode_paged,
    decode_paged_fp8,
    decode_workspace_size,
    load_library,
    new_decode_workspace,
    prefill,
)
