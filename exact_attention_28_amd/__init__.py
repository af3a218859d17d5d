"""MI355X (gfx950) exact attention: fused forward, backward and paged decode.

The computation lives in ``libfa.so`` (hand-written HIP kernels behind the
C ABI of ``include/fa.h``); this package only binds it. Build it in-tree
with ``python -m exact_attention_28_amd.build``.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    FA_DTYPE_BF16,
    FA_DTYPE_F32,
    FA_DTYPE_FP8_E4M3,
    FaError,
    LIB_PATH,
    fa_bwd,
    fa_bwd_workspace_size,
    fa_fwd,
    fa_naive_attention,
    fa_naive_workspace_size,
    fa_paged_decode,
    fa_paged_decode_fp8kv,
    fa_paged_decode_noalloc,
    fa_paged_decode_workspace_size,
    fa_paged_prefill,
    fa_strerror,
    load_library,
)
from .api import attention, attention_backward, paged_decode  # noqa: F401
