"""ctypes binding of libfa.so: same names and arguments as include/fa.h.

Argument marshalling only: tensors are passed as device pointers
(``data_ptr()``), sizes as ints, the stream as a hipStream_t handle. Every
step of the computation runs in the library's HIP kernels. There is no
fallback: if libfa.so is missing, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_FP8_E4M3 = 2

FA_OK = 0
FA_EINVAL_NULL = -1
FA_EINVAL_DIM = -2
FA_EUNSUPPORTED_D = -3
FA_EGQA = -4
FA_EDTYPE = -5
FA_EDESCALE = -6
FA_ESCALE = -7
FA_EPAGE = -8
FA_EWORKSPACE = -9
FA_ESPLITS = -10
FA_EALIGN = -11
FA_ESCRATCH = -12

# every function include/fa.h declares
EXPORTS = ("fa_fwd", "fa_bwd", "fa_bwd_workspace_size", "fa_naive_attention",
           "fa_naive_workspace_size", "fa_paged_decode",
           "fa_paged_decode_fp8kv", "fa_paged_decode_noalloc",
           "fa_paged_decode_workspace_size",
           "fa_paged_prefill", "fa_strerror")


class FaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{message} (code {code})")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libfa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FaError(-1000, f"{path} not built: run "
                      "`python -m exact_attention_28_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.restype = i
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i,
                           vp, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd.argtypes = [vp] * 9 + [i] * 6 + [f, i, i, vp, sz, vp]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_bwd_workspace_size.argtypes = [i, i, i]
    lib.fa_paged_decode.restype = i
    lib.fa_paged_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i,
                                    f, vp, vp, vp, sz, i, vp]
    lib.fa_paged_prefill.restype = i
    lib.fa_paged_prefill.argtypes = [vp] * 5 + [i] * 8 + [f, i, vp, vp, vp]
    lib.fa_naive_attention.restype = i
    lib.fa_naive_attention.argtypes = [vp] * 5 + [i] * 6 + [f, i, vp, sz, vp]
    lib.fa_naive_workspace_size.restype = sz
    lib.fa_naive_workspace_size.argtypes = [i, i, i, i]
    lib.fa_paged_decode_noalloc.restype = i
    lib.fa_paged_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i,
                                            i, i, i, f, vp, vp, i, vp]
    lib.fa_paged_decode_fp8kv.restype = i
    lib.fa_paged_decode_fp8kv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i,
                                          i, i, f, vp, vp, vp, vp, sz, i, vp]
    lib.fa_paged_decode_workspace_size.restype = sz
    lib.fa_paged_decode_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_strerror.argtypes = [i]
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()          # torch tensor (device memory)


def _stream(s, *tensors):
    """hipStream_t handle: the given stream, else torch's current stream of
    the first device tensor, else NULL (the default stream)."""
    if s is not None:
        return s if isinstance(s, int) else s.cuda_stream
    for t in tensors:
        if getattr(t, "is_cuda", False):
            import torch
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _check(code: int):
    if code != FA_OK:
        raise FaError(code, fa_strerror(code))


def fa_strerror(code: int) -> str:
    return load_library().fa_strerror(int(code)).decode()


def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype,
           qkv_descale=None, stream=None, check=True) -> int:
    """Exact attention forward (see include/fa.h). qkv_descale: three floats
    (host values) or None. Returns the library's code; raises FaError on a
    non-zero code unless check=False."""
    lib = load_library()
    desc = None
    if qkv_descale is not None:
        desc = (ctypes.c_float * 3)(*[float(x) for x in qkv_descale])
    code = lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                      int(B), int(Hq), int(Hkv), int(Nq), int(Nk), int(d),
                      float(scale), int(bool(causal)), int(dtype),
                      ctypes.cast(desc, ctypes.c_void_p) if desc else None,
                      _stream(stream, q, o))
    if check:
        _check(code)
    return code


def fa_bwd_workspace_size(B, Hq, Nq) -> int:
    return int(load_library().fa_bwd_workspace_size(int(B), int(Hq), int(Nq)))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale,
           causal, dtype, workspace, workspace_bytes, stream=None,
           check=True) -> int:
    """Exact attention backward (see include/fa.h)."""
    lib = load_library()
    code = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                      _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), int(B),
                      int(Hq), int(Hkv), int(Nq), int(Nk), int(d),
                      float(scale), int(bool(causal)), int(dtype),
                      _ptr(workspace), int(workspace_bytes),
                      _stream(stream, q, dq))
    if check:
        _check(code)
    return code


def fa_paged_decode_workspace_size(B, Hq, Hkv, d, max_pages_per_seq,
                                   page_size, num_splits=0) -> int:
    return int(load_library().fa_paged_decode_workspace_size(
        int(B), int(Hq), int(Hkv), int(d), int(max_pages_per_seq),
        int(page_size), int(num_splits)))


def fa_paged_decode(q, k_pool, v_pool, block_table, seq_lens, page_size,
                    num_pages, B, Hq, Hkv, d, max_pages_per_seq, scale, o,
                    lse, workspace, workspace_bytes, num_splits=0,
                    stream=None, check=True) -> int:
    """Paged-KV decode (see include/fa.h)."""
    lib = load_library()
    code = lib.fa_paged_decode(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
        _ptr(seq_lens), int(page_size), int(num_pages), int(B), int(Hq),
        int(Hkv), int(d), int(max_pages_per_seq), float(scale), _ptr(o),
        _ptr(lse), _ptr(workspace), int(workspace_bytes), int(num_splits),
        _stream(stream, q, o))
    if check:
        _check(code)
    return code


def fa_paged_decode_noalloc(q, k_pool, v_pool, block_table, seq_lens,
                            page_size, num_pages, B, Hq, Hkv, d,
                            max_pages_per_seq, scale, o, lse, num_splits=0,
                            stream=None, check=True) -> int:
    """Paged-KV decode with the library's built-in workspace (see
    include/fa.h): nothing is allocated by the call."""
    lib = load_library()
    code = lib.fa_paged_decode_noalloc(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
        _ptr(seq_lens), int(page_size), int(num_pages), int(B), int(Hq),
        int(Hkv), int(d), int(max_pages_per_seq), float(scale), _ptr(o),
        _ptr(lse), int(num_splits), _stream(stream, q, o))
    if check:
        _check(code)
    return code


def fa_paged_decode_fp8kv(q, k_pool, v_pool, block_table, seq_lens,
                          page_size, num_pages, B, Hq, Hkv, d,
                          max_pages_per_seq, scale, kv_descale, o, lse,
                          workspace, workspace_bytes, num_splits=0,
                          stream=None, check=True) -> int:
    """Paged decode over an e4m3 cache (see include/fa.h). kv_descale: two
    floats (s_k, s_v) on the host, or None."""
    lib = load_library()
    desc = None
    if kv_descale is not None:
        desc = (ctypes.c_float * 2)(*[float(x) for x in kv_descale])
    code = lib.fa_paged_decode_fp8kv(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
        _ptr(seq_lens), int(page_size), int(num_pages), int(B), int(Hq),
        int(Hkv), int(d), int(max_pages_per_seq), float(scale),
        ctypes.cast(desc, ctypes.c_void_p) if desc else None, _ptr(o),
        _ptr(lse), _ptr(workspace), int(workspace_bytes), int(num_splits),
        _stream(stream, q, o))
    if check:
        _check(code)
    return code


def fa_naive_workspace_size(B, Hq, Nq, Nk) -> int:
    return int(load_library().fa_naive_workspace_size(int(B), int(Hq),
                                                      int(Nq), int(Nk)))


def fa_naive_attention(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                       workspace, workspace_bytes, stream=None,
                       check=True) -> int:
    """The three-kernel contrast path (see include/fa.h)."""
    code = load_library().fa_naive_attention(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(Hq),
        int(Hkv), int(Nq), int(Nk), int(d), float(scale), int(bool(causal)),
        _ptr(workspace), int(workspace_bytes), _stream(stream, q, o))
    if check:
        _check(code)
    return code


def fa_paged_prefill(q, k_pool, v_pool, block_table, seq_lens, page_size,
                     num_pages, B, Hq, Hkv, Nq, d, max_pages_per_seq, scale,
                     causal, o, lse, stream=None, check=True) -> int:
    """Chunked prefill against a paged cache (see include/fa.h)."""
    code = load_library().fa_paged_prefill(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
        _ptr(seq_lens), int(page_size), int(num_pages), int(B), int(Hq),
        int(Hkv), int(Nq), int(d), int(max_pages_per_seq), float(scale),
        int(bool(causal)), _ptr(o), _ptr(lse), _stream(stream, q, o))
    if check:
        _check(code)
    return code
