"""The tensor-level API checks every tensor before it reaches the C ABI
(which sees only addresses and sizes): CPU tensors, int64 tables, mixed
dtypes and wrong shapes raise FaError and launch nothing. Runs without a
GPU: every call below is refused before the library is called."""
import pytest
import torch

import exact_attention_28_amd as fa
from exact_attention_28_amd import api

bf = torch.bfloat16


def _qkv(dtype=bf, B=1, Hq=4, Hkv=2, N=32, d=64):
    q = torch.zeros((B, Hq, N, d), dtype=dtype)
    k = torch.zeros((B, Hkv, N, d), dtype=dtype)
    v = torch.zeros((B, Hkv, N, d), dtype=dtype)
    return q, k, v


def _raises(fn, *a, match, **kw):
    with pytest.raises(fa.FaError, match=match) as e:
        fn(*a, **kw)
    assert e.value.code == api.TENSOR_CHECK


def test_forward_cpu_tensors_rejected():
    q, k, v = _qkv()
    _raises(fa.attention, q, k, v, match="not in GPU memory")


def test_forward_mixed_dtypes_rejected():
    q, k, v = _qkv()
    _raises(fa.attention, q.float(), k, v, match="k: dtype")
    _raises(fa.attention, q, k, v.float(), match="v: dtype")


def test_forward_shapes_rejected():
    q, k, v = _qkv()
    _raises(fa.attention, q, k, v[:, :, :16].contiguous(), match="v: shape")
    _raises(fa.attention, q, k[..., :32].contiguous(), v, match="k: shape")
    _raises(fa.attention, q, k, v, out=torch.zeros((1, 4, 32, 64)),
            match="out: dtype")
    _raises(fa.attention, q, k, v, lse=torch.zeros((1, 4, 31)),
            match="lse: shape")
    _raises(fa.attention, q[0], k[0], v[0], match="expected")


def _cache(B=3, Hq=8, Hkv=2, d=64, pages=10, max_pages=4):
    q = torch.zeros((B, Hq, d), dtype=bf)
    kp = torch.zeros((pages, 16, Hkv, d), dtype=bf)
    vp = torch.zeros((pages, 16, Hkv, d), dtype=bf)
    bt = torch.zeros((B, max_pages), dtype=torch.int32)
    sl = torch.full((B,), 20, dtype=torch.int32)
    return q, kp, vp, bt, sl


def test_decode_int64_tables_rejected():
    q, kp, vp, bt, sl = _cache()
    _raises(fa.paged_decode, q, kp, vp, bt.long(), sl,
            match="block_table: dtype")
    _raises(fa.paged_decode, q, kp, vp, bt, sl.long(), match="seq_lens: dtype")
    # a table built from a Python list defaults to int64
    _raises(fa.paged_decode, q, kp, vp, torch.tensor([[0], [1], [2]]), sl,
            match="block_table: dtype")


def test_decode_shapes_and_dtypes_rejected():
    q, kp, vp, bt, sl = _cache()
    _raises(fa.paged_decode, q.float(), kp, vp, bt, sl, match="q: dtype")
    _raises(fa.paged_decode, q, kp, vp.float(), bt, sl, match="v_pool: dtype")
    _raises(fa.paged_decode, q, kp, vp[:5].contiguous(), bt, sl,
            match="v_pool: shape")
    _raises(fa.paged_decode, q, kp, vp, bt[:2].contiguous(), sl,
            match="block_table: shape")
    _raises(fa.paged_decode, q, kp, vp, bt, sl[:2].contiguous(),
            match="seq_lens: shape")
    _raises(fa.paged_decode, q[..., :32].contiguous(), kp, vp, bt, sl,
            match="head dim")
    _raises(fa.paged_decode, q, kp, vp, bt, sl,
            workspace=torch.zeros(16, dtype=torch.float32),
            match="workspace: dtype")


def test_decode_cpu_tensors_rejected():
    q, kp, vp, bt, sl = _cache()
    _raises(fa.paged_decode, q, kp, vp, bt, sl, match="not in GPU memory")


def test_backward_checks():
    q, k, v = _qkv()
    o = torch.zeros_like(q)
    g = torch.zeros_like(q)
    lse = torch.zeros((1, 4, 32), dtype=torch.float32)
    _raises(fa.attention_backward, q, k, v, o, lse, g.float(),
            match="dout: dtype")
    _raises(fa.attention_backward, q, k, v, o, lse.double(), g,
            match="lse: dtype")
    _raises(fa.attention_backward, q, k, v, o[:, :2].contiguous(), lse, g,
            match="o: shape")
    _raises(fa.attention_backward, q, k, v, o, lse, g,
            match="not in GPU memory")
