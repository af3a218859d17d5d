"""HIP graph capture of the entry points through the C ABI.

The forward, the backward and the paged decode allocate nothing and record
no memset (the decode's bookkeeping is written by its own kernel), so a
caller may capture them into a graph, as a serving or training loop does.
One graph holds a causal GQA forward, its backward and a paged decode; it is
replayed several times with unrelated eager work and synchronisations in
between, the outputs cleared before each replay, and every replay must equal
the eager result bit for bit (the kernels are deterministic).
"""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_28_amd as m
    m.load_library()
    return m


def test_graph_replays_match_eager(fa):
    dev = torch.device("cuda:0")
    print("graph capture: fwd + bwd + decode", flush=True)
    inp = W.prefill_inputs(1, 8, 2, 600, 600, 128, dtype="bf16", causal=True,
                           seed=3)
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    do = W.upstream_grad((1, 8, 600, 128), seed=4).to(dev)
    di = W.decode_inputs(12, 8, 2, 128, lens=[1, 16, 17, 300, 512, 1000, 33,
                                              64, 2048, 5, 700, 129],
                         max_pages=128, seed=5)
    dq_, kp, vp = (t.to(dev) for t in (di.q, di.k_pool, di.v_pool))
    bt, sl = di.block_table.to(dev), di.seq_lens.to(dev)
    ws_b = torch.empty(fa.fa_bwd_workspace_size(1, 8, 600), dtype=torch.uint8,
                       device=dev)
    ws_d = torch.empty(fa.fa_paged_decode_workspace_size(12, 8, 2, 128, 128,
                                                         16, 0),
                       dtype=torch.uint8, device=dev)

    def run(outs):
        o, l, gq, gk, gv, od, ld = outs
        fa.attention(q, k, v, causal=True, scale=inp.scale, out=o, lse=l)
        fa.attention_backward(q, k, v, o, l, do, causal=True, scale=inp.scale,
                              dq=gq, dk=gk, dv=gv, workspace=ws_b)
        fa.paged_decode(dq_, kp, vp, bt, sl, scale=di.scale, out=od, lse=ld,
                        workspace=ws_d)

    def alloc():
        return [torch.empty((1, 8, 600, 128), dtype=torch.bfloat16, device=dev),
                torch.empty((1, 8, 600), dtype=torch.float32, device=dev),
                torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                torch.empty((12, 8, 128), dtype=torch.bfloat16, device=dev),
                torch.empty((12, 8), dtype=torch.float32, device=dev)]

    eager = alloc()
    run(eager)
    torch.cuda.synchronize()

    static = alloc()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(static)  # warm-up on the capture stream's side, as torch advises
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(static)
    torch.cuda.synchronize()

    a = torch.randn(512, 512, device=dev)
    for rep in range(4):
        for t in static:
            t.zero_()
        _ = (a @ a).sum().item()  # unrelated eager work and a sync
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("O", "LSE", "dQ", "dK", "dV", "decode O",
                               "decode LSE"), static, eager):
            assert torch.equal(x, y), f"replay {rep}: {name} differs"
