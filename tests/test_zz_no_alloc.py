"""fa_paged_decode_noalloc (the decode with the library's built-in
workspace) against fa_paged_decode (caller workspace), both through the C
ABI on the same seeded inputs.

Two calls in a row, the second with a smaller input, so the second reads a
workspace that still holds the first call's partials; then a batch large
enough that the automatic range count has to be lowered to fit the
built-in workspace. Where both entry points run the same plan they launch
the same kernels on the same inputs, so the outputs must be bit-identical;
a lowered range count changes only the fp32 summation order, and is held
to the bf16 bars (O <= 1e-2, LSE <= 1e-3)."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 16 << 20


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_28_amd as m
    m.load_library()
    return m


def _run(fa, di, num_splits=0):
    dev = torch.device("cuda:0")
    q = di.q.to(dev)
    kp, vp = di.k_pool.to(dev), di.v_pool.to(dev)
    bt, sl = di.block_table.to(dev), di.seq_lens.to(dev)
    B, Hq, d = q.shape
    npages, page, Hkv, _ = kp.shape
    maxp = bt.shape[1]
    need = fa.fa_paged_decode_workspace_size(B, Hq, Hkv, d, maxp, page,
                                             num_splits)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    o_ref = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev)
    l_ref = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    fa.fa_paged_decode(q, kp, vp, bt, sl, page, npages, B, Hq, Hkv, d, maxp,
                       di.scale, o_ref, l_ref, ws, need, num_splits)
    o = torch.empty_like(o_ref)
    lse = torch.empty_like(l_ref)
    fa.fa_paged_decode_noalloc(q, kp, vp, bt, sl, page, npages, B, Hq, Hkv,
                               d, maxp, di.scale, o, lse, num_splits)
    torch.cuda.synchronize()
    return (o.double().cpu().numpy(), lse.double().cpu().numpy(),
            o_ref.double().cpu().numpy(), l_ref.double().cpu().numpy(), need)


def _max_err(a, b):
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    assert np.array_equal(a[~fin], b[~fin])
    return float(np.max(np.abs(a[fin] - b[fin]), initial=0.0))


def test_noalloc_two_calls_second_smaller(fa):
    # first: the full decode workload (64 requests, L ~ U{512..8192},
    # Hq 32, Hkv 8, d 128); second: 5 short requests, Hq 8, Hkv 2, d 64
    first = W.decode_config("paged_decode_r64_hq32_hkv8_d128_p16")
    second = W.decode_inputs(5, 8, 2, 64, lens=[1, 16, 17, 300, 0], seed=7,
                             max_pages=32)
    for name, di in (("decode 64 req d128", first), ("5 req d64", second)):
        print(f"noalloc vs workspace decode: {name}", flush=True)
        o, lse, ro, rl, need = _run(fa, di)
        assert need <= SCRATCH_BYTES   # same plan on both sides
        assert np.array_equal(o, ro), name
        assert np.array_equal(lse, rl), name


def test_noalloc_lowered_range_count(fa):
    # 1000 short requests: the automatic plan's partials exceed the 16 MiB
    # built-in workspace, so the no-alloc call runs fewer ranges
    lens = np.random.default_rng(11).integers(1, 200, size=1000, endpoint=True)
    di = W.decode_inputs(1000, 32, 8, 128, lens=list(lens), seed=11,
                         max_pages=16)
    print("noalloc vs workspace decode: 1000 req (lowered ranges)", flush=True)
    o, lse, ro, rl, need = _run(fa, di)
    assert need > SCRATCH_BYTES
    eo, el = _max_err(o, ro), _max_err(lse, rl)
    print(f"  max|dO|={eo:.2e} max|dLSE|={el:.2e}", flush=True)
    assert eo <= 1e-2 and el <= 1e-3


def test_noalloc_explicit_split_too_large_rejected(fa):
    di = W.decode_inputs(4, 8, 2, 128, lens=[100, 200, 300, 400], seed=3,
                         max_pages=32)
    dev = torch.device("cuda:0")
    o = torch.full((4, 8, 128), 7.0, dtype=torch.bfloat16, device=dev)
    lse = torch.full((4, 8), 7.0, dtype=torch.float32, device=dev)
    code = fa.fa_paged_decode_noalloc(
        di.q.to(dev), di.k_pool.to(dev), di.v_pool.to(dev),
        di.block_table.to(dev), di.seq_lens.to(dev), 16, di.k_pool.shape[0],
        4, 8, 2, 128, 32, di.scale, o, lse, 65536, check=False)
    torch.cuda.synchronize()
    assert code == fa._lib.FA_ESCRATCH
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
