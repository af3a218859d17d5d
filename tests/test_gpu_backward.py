"""GPU parity of the backward pass (fa_bwd, through the C ABI) against the
fp64 oracle's gradient of the definition, on the same seeded bf16 inputs.

The GPU path takes O and LSE from its own bf16 forward (as a training step
does) and re-computes P from them; the oracle differentiates the definition
on the same bf16-rounded Q, K, V and dO in fp64.

Bar, per gradient tensor: max |g - g_ref| <= 1e-2 * max |g_ref| + 1e-3.
Where it comes from: every gradient element is rounded once to bf16
(relative 2^-9 = 0.2 %); P and dS enter their products as bf16 (relative
2^-9 per element, averaging out over the summed rows or keys); D =
rowsum(dO * O) uses the bf16 O of the forward. Together these stay well
under 1 % of the tensor's largest element; the absolute floor covers
tensors whose entries are all tiny (short causal rows).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

RTOL, ATOL = 1e-2, 1e-3


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_28_amd as m
    m.load_library()
    return m


def _run(fa, B, Hq, Hkv, Nq, Nk, d, causal, seed):
    inp = W.prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dtype="bf16",
                           causal=causal, seed=seed)
    g = W.upstream_grad((B, Hq, Nq, d), seed=seed + 1000)
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in (inp.q, inp.k, inp.v, g))
    print(f"bwd case B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} "
          f"causal={causal} seed={seed}", flush=True)
    o, lse = fa.attention(q, k, v, causal=causal, scale=inp.scale)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, causal=causal,
                                       scale=inp.scale)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(W.as_f64(inp.q), W.as_f64(inp.k),
                                    W.as_f64(inp.v), W.as_f64(g), inp.scale,
                                    causal=causal)
    out = [t.double().cpu().numpy() for t in (dq, dk, dv)]
    return out, ref


def _check(out, ref, what, names=("dQ", "dK", "dV")):
    for name, a, r in zip(names, out, ref):
        assert not np.any(np.isnan(a)), f"{what} {name} NaN"
        err = float(np.max(np.abs(a - r)))
        bound = RTOL * float(np.max(np.abs(r))) + ATOL
        print(f"  {name}: max|err| {err:.3e}  max|ref| {np.max(np.abs(r)):.3e}"
              f"  bound {bound:.3e}", flush=True)
        assert err <= bound, (what, name, err, bound)


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal", [
    (1, 1, 1, 64, 64, 64, False),
    (1, 2, 2, 200, 200, 128, False),     # ragged tails
    (1, 2, 2, 200, 200, 128, True),
    (2, 4, 2, 256, 256, 128, True),      # GQA
    (1, 4, 1, 130, 130, 64, True),       # GQA 4:1, d = 64, ragged
    (1, 2, 1, 96, 300, 128, True),       # Nk > Nq (bottom-right causal)
    (1, 2, 2, 300, 96, 128, True),       # Nq > Nk: early rows see no key
    (1, 2, 2, 333, 257, 64, False),
    (3, 6, 2, 150, 200, 128, True),      # odd group size, B = 3
    (1, 2, 1, 1000, 1100, 128, True),    # many interior and diagonal tiles
])
def test_backward_matches_oracle(fa, B, Hq, Hkv, Nq, Nk, d, causal):
    out, ref = _run(fa, B, Hq, Hkv, Nq, Nk, d, causal, seed=Nq + Nk + d)
    _check(out, ref, f"bwd {B}x{Hq}/{Hkv}x{Nq}x{Nk}x{d} causal={causal}")


def test_backward_several_dispatch_rounds(fa):
    # more workgroups than the GPU runs at once (dK/dV: 1024 of 128 keys,
    # dQ: 2048 of 128 rows, both two to a CU), so the later dispatch rounds
    # walk their tiles the other way; every gradient compared in full
    out, ref = _run(fa, 16, 32, 16, 512, 512, 128, True, seed=31)
    _check(out, ref, "bwd 16x32/16x512x512x128 causal, several rounds")


def test_backward_rows_without_keys_are_zero(fa):
    out, ref = _run(fa, 1, 2, 2, 300, 96, 64, True, seed=5)
    dq = out[0]
    assert np.all(dq[:, :, : 300 - 96] == 0)


def test_backward_is_deterministic(fa):
    a, _ = _run(fa, 1, 4, 2, 256, 256, 128, True, seed=9)
    b, _ = _run(fa, 1, 4, 2, 256, 256, 128, True, seed=9)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_long_causal_sampled(fa):
    # a long causal GQA problem: dQ rows and dK/dV keys sampled against the
    # oracle restricted to the rows and keys they depend on
    B, Hq, Hkv, N, d = 1, 4, 1, 4096, 128
    inp = W.prefill_inputs(B, Hq, Hkv, N, N, d, dtype="bf16", causal=True,
                           seed=77)
    g = W.upstream_grad((B, Hq, N, d), seed=78)
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in (inp.q, inp.k, inp.v, g))
    o, lse = fa.attention(q, k, v, causal=True, scale=inp.scale)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, causal=True,
                                       scale=inp.scale)
    torch.cuda.synchronize()
    # The last 96 rows against every key (bottom-right causal alignment
    # keeps each row's own key range): that gives their dQ exactly, and the
    # dK, dV of the last 96 keys, which no earlier row can see.
    n = 96
    gs = W.as_f64(g)[:, :, N - n:]
    full = oracle.attention_backward(
        W.as_f64(inp.q)[:, :, N - n:], W.as_f64(inp.k), W.as_f64(inp.v), gs,
        inp.scale, causal=True)
    dq_ref = full[0]
    dk_ref = full[1][:, :, N - n:]
    dv_ref = full[2][:, :, N - n:]
    out = [dq.double().cpu().numpy()[:, :, N - n:],
           dk.double().cpu().numpy()[:, :, N - n:],
           dv.double().cpu().numpy()[:, :, N - n:]]
    _check(out, (dq_ref, dk_ref, dv_ref), "long causal corner")


def test_backward_full_workload_sampled(fa):
    # the causal GQA prefill at full size (B=1, Hq=32, Hkv=8, N=16384,
    # d=128, the shape and launch the benchmark times), dO from seed 43:
    # dQ of the first, a middle and the last 64 rows, each against the
    # oracle on the key prefix those rows can see (so the bottom-right
    # alignment of the sliced problem is the true one), and dK, dV of the
    # last 64 keys, which only the last 64 rows see
    name = "bf16_causal_gqa_b1_hq32_hkv8_n16384_d128"
    c = W.PREFILL_CONFIGS[name]
    inp = W.prefill_config(name)
    N = c["Nq"]
    g = W.upstream_grad(tuple(inp.q.shape), seed=43)
    dev = torch.device("cuda:0")
    print(f"bwd full workload {name}", flush=True)
    q, k, v, do = (t.to(dev) for t in (inp.q, inp.k, inp.v, g))
    o, lse = fa.attention(q, k, v, causal=True, scale=inp.scale)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, causal=True,
                                       scale=inp.scale)
    torch.cuda.synchronize()
    dq = dq.double().cpu().numpy()
    dk = dk.double().cpu().numpy()
    dv = dv.double().cpu().numpy()
    q64, k64, v64, g64 = (W.as_f64(t) for t in (inp.q, inp.k, inp.v, g))
    n = 64
    for r0 in (0, N // 2 + 37, N - n):
        ref = oracle.attention_backward(q64[:, :, r0:r0 + n],
                                        k64[:, :, :r0 + n], v64[:, :, :r0 + n],
                                        g64[:, :, r0:r0 + n], inp.scale,
                                        causal=True)
        _check([dq[:, :, r0:r0 + n]], [ref[0]], f"full workload dQ rows {r0}..")
        if r0 == N - n:
            _check([dk[:, :, r0:], dv[:, :, r0:]],
                   [ref[1][:, :, r0:], ref[2][:, :, r0:]],
                   "full workload dK, dV of the last keys", names=("dK", "dV"))


@pytest.mark.parametrize("d", [64, 128])
def test_backward_workspace_contents_do_not_matter(fa, d):
    # Nq not a multiple of the 32-row tile: the last query tile of the last
    # head reads the workspace rows after the real ones. The workspace is
    # filled with NaN bytes first; the gradients must not see them.
    B, Hq, Hkv, N, causal = 1, 2, 1, 200, True
    inp = W.prefill_inputs(B, Hq, Hkv, N, N, d, dtype="bf16", causal=causal,
                           seed=77 + d)
    g = W.upstream_grad((B, Hq, N, d), seed=78 + d)
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in (inp.q, inp.k, inp.v, g))
    print(f"bwd NaN-filled workspace d={d}", flush=True)
    o, lse = fa.attention(q, k, v, causal=causal, scale=inp.scale)
    need = fa.fa_bwd_workspace_size(B, Hq, N)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, causal=causal,
                                       scale=inp.scale, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(W.as_f64(inp.q), W.as_f64(inp.k),
                                    W.as_f64(inp.v), W.as_f64(g), inp.scale,
                                    causal=causal)
    out = [t.double().cpu().numpy() for t in (dq, dk, dv)]
    _check(out, ref, f"bwd NaN-filled workspace d={d}")
