"""Tensor-level convenience over the C ABI: allocate outputs with torch,
read shapes off the tensors, call libfa. No arithmetic happens here."""
from __future__ import annotations

import math

from . import _lib


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return _lib.FA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return _lib.FA_DTYPE_BF16
    if t.dtype == torch.float8_e4m3fn:
        return _lib.FA_DTYPE_FP8_E4M3
    raise _lib.FaError(_lib.FA_EDTYPE, f"unsupported dtype {t.dtype}")


def attention(q, k, v, causal=False, scale=None, descale=None, out=None,
              lse=None, stream=None, want_lse=True):
    """O, LSE = exact attention of device tensors q [B,Hq,Nq,d], k/v
    [B,Hkv,Nk,d] (fp32, bf16, or float8_e4m3fn with descale=(s_q,s_k,s_v))."""
    import torch
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    odt = torch.float32 if code == _lib.FA_DTYPE_F32 else torch.bfloat16
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
    B, Hq, d = q.shape
    num_pages, page_size, Hkv, _ = k_pool.shape
    max_pages = block_table.shape[1]
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
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
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
