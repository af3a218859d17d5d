"""fp64 CPU oracle for exact attention (forward and backward) and paged decode.

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product path.
"""
from .attention import (  # noqa: F401
    attention,
    attention_backward,
    attention_fp8,
    attention_fp8_p_e4m3,
    gather_paged_kv,
    merge_partials,
    online_softmax_stats,
    paged_decode,
    paged_decode_fp8,
    paged_prefill,
    round_e4m3,
    safe_softmax,
    softmax_stats,
)
