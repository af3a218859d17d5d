"""Tensor-level convenience over the C ABI: allocate outputs with torch,
read shapes off the tensors, call libfa. No arithmetic happens here.

The C ABI sees only addresses and sizes, so every tensor is checked here
before the call: its dtype and shape against the others', then that it is
contiguous device memory on the same GPU as the query. A mismatch raises
FaError with code TENSOR_CHECK (a Python-side code, not one of the
library's) and nothing is launched."""
from __future__ import annotations

import math

from . import _lib

TENSOR_CHECK = -1001


def _fail(msg):
    raise _lib.FaError(TENSOR_CHECK, msg)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return _lib.FA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return _lib.FA_DTYPE_BF16
    if t.dtype == torch.float8_e4m3fn:
        return _lib.FA_DTYPE_FP8_E4M3
    raise _lib.FaError(_lib.FA_EDTYPE, f"unsupported dtype {t.dtype}")


def _expect(name, t, dtype, shape):
    """dtype and shape of one tensor (checked before the device)."""
    if t.dtype != dtype:
        _fail(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        _fail(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _on_device(dev, **tensors):
    """Every tensor contiguous, in GPU memory, on the query's device."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not getattr(t, "is_cuda", False):
            _fail(f"{name}: not in GPU memory (device {t.device})")
        if t.device != dev:
            _fail(f"{name}: on {t.device}, the query is on {dev}")
        if not t.is_contiguous():
            _fail(f"{name}: not contiguous")


def _workspace_ok(name, ws):
    import torch
    if ws is not None and ws.dtype != torch.uint8:
        _fail(f"{name}: dtype {ws.dtype}, expected torch.uint8")


def _paged_cache(q, k_pool, v_pool, block_table, seq_lens, pool_dtype):
    """Shapes of a paged cache and its table; returns
    (num_pages, page_size, Hkv, max_pages)."""
    import torch
    if k_pool.dim() != 4:
        _fail(f"k_pool: {k_pool.dim()} dims, expected [num_pages, page_size, Hkv, d]")
    num_pages, page_size, Hkv, dk = k_pool.shape
    _expect("k_pool", k_pool, pool_dtype, k_pool.shape)
    _expect("v_pool", v_pool, pool_dtype, k_pool.shape)
    if dk != q.shape[-1]:
        _fail(f"k_pool: head dim {dk}, the query's is {q.shape[-1]}")
    if block_table.dim() != 2:
        _fail("block_table: expected [B, max_pages_per_seq]")
    B = q.shape[0]
    _expect("block_table", block_table, torch.int32, (B, block_table.shape[1]))
    _expect("seq_lens", seq_lens, torch.int32, (B,))
    return num_pages, page_size, Hkv, block_table.shape[1]


def attention(q, k, v, causal=False, scale=None, descale=None, out=None,
              lse=None, stream=None, want_lse=True):
    """O, LSE = exact attention of device tensors q [B,Hq,Nq,d], k/v
    [B,Hkv,Nk,d] (fp32, bf16, or float8_e4m3fn with descale=(s_q,s_k,s_v))."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        _fail("q, k, v: expected [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    code = _dtype_code(q)
    _expect("k", k, q.dtype, (B, Hkv, Nk, d))
    _expect("v", v, q.dtype, (B, Hkv, Nk, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    odt = torch.float32 if code == _lib.FA_DTYPE_F32 else torch.bfloat16
    if out is not None:
        _expect("out", out, odt, (B, Hq, Nq, d))
    if lse is not None:
        _expect("lse", lse, torch.float32, (B, Hq, Nq))
    _on_device(q.device, q=q, k=k, v=v, out=out, lse=lse)
    if out is None:
        out = torch.empty((B, Hq, Nq, d), dtype=odt, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _lib.fa_fwd(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                code, descale, stream)
    return out, lse


def paged_decode(q, k_pool, v_pool, block_table, seq_lens, scale=None,
                 num_splits=0, out=None, lse=None, workspace=None,
                 stream=None):
    """O [B,Hq,d] bf16, LSE [B,Hq] for one query token per request."""
    import torch
    if q.dim() != 3:
        _fail("q: expected [B, Hq, d]")
    B, Hq, d = q.shape
    _expect("q", q, torch.bfloat16, q.shape)
    num_pages, page_size, Hkv, max_pages = _paged_cache(
        q, k_pool, v_pool, block_table, seq_lens, torch.bfloat16)
    if out is not None:
        _expect("out", out, torch.bfloat16, (B, Hq, d))
    if lse is not None:
        _expect("lse", lse, torch.float32, (B, Hq))
    _workspace_ok("workspace", workspace)
    _on_device(q.device, q=q, k_pool=k_pool, v_pool=v_pool,
               block_table=block_table, seq_lens=seq_lens, out=out, lse=lse,
               workspace=workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = _lib.fa_paged_decode_workspace_size(B, Hq, Hkv, d, max_pages,
                                               page_size, num_splits)
    if (workspace is None or
            workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _lib.fa_paged_decode(q, k_pool, v_pool, block_table, seq_lens, page_size,
                         num_pages, B, Hq, Hkv, d, max_pages, scale, out,
                         lse, workspace,
                         workspace.numel() * workspace.element_size(),
                         num_splits, stream)
    return out, lse


def attention_backward(q, k, v, o, lse, dout, causal=False, scale=None,
                       dq=None, dk=None, dv=None, workspace=None,
                       stream=None):
    """dQ, dK, dV (bf16) of exact attention, from the forward's o and lse
    and the upstream gradient dout; P is re-computed in the kernels."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        _fail("q, k, v: expected [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    bf = torch.bfloat16
    _expect("q", q, bf, q.shape)
    for name, t in (("k", k), ("v", v), ("dk", dk), ("dv", dv)):
        if t is not None:
            _expect(name, t, bf, (B, Hkv, Nk, d))
    for name, t in (("o", o), ("dout", dout), ("dq", dq)):
        if t is not None:
            _expect(name, t, bf, (B, Hq, Nq, d))
    _expect("lse", lse, torch.float32, (B, Hq, Nq))
    _workspace_ok("workspace", workspace)
    _on_device(q.device, q=q, k=k, v=v, o=o, lse=lse, dout=dout, dq=dq,
               dk=dk, dv=dv, workspace=workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = _lib.fa_bwd_workspace_size(B, Hq, Nq)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8,
                                device=q.device)
    _lib.fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d,
                scale, causal, _dtype_code(q), workspace,
                workspace.numel() * workspace.element_size(), stream)
    return dq, dk, dv
