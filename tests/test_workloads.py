"""The seeded generators: number formats, determinism and cache structure.

bf16 must be round-to-nearest-even of the fp32 draw; e4m3 is OCP e4m3fn
(bias 7, largest finite 448, smallest subnormal 2^-9) with ties to even,
after a per-tensor scale that maps the largest magnitude to 448. These are
checked against values fixed by the formats' definitions.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W


def _bf16(xs):
    t, _ = W._to_storage(np.array(xs, dtype=np.float32), "bf16")
    return t.to(torch.float64).numpy()


def test_bf16_round_to_nearest_even():
    u = 2.0 ** -7                    # bf16 ulp at 1.0
    got = _bf16([1.0 + u / 2, 1.0 + 1.5 * u, 1.0 + 0.51 * u, -1.0 - u / 2,
                 3.0e38, 2.0 ** -133])
    assert got[0] == 1.0                  # tie -> even (mantissa 0)
    assert got[1] == 1.0 + 2 * u          # tie -> even (mantissa 2)
    assert got[2] == 1.0 + u              # above the tie -> up
    assert got[3] == -1.0                 # sign symmetric
    assert got[4] == float(np.float32(3.0e38)) or math.isfinite(got[4])
    assert got[5] == 2.0 ** -133          # bf16 keeps fp32 subnormal range


def _e4m3_values():
    """All finite non-negative OCP e4m3fn values, from the definition."""
    vals = set()
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue                  # the NaN code
            if e == 0:
                vals.add(m * 2.0 ** -9)   # subnormals: m/8 * 2^-6
            else:
                vals.add((1 + m / 8) * 2.0 ** (e - 7))
    return np.array(sorted(vals))


def test_e4m3_grid_and_rounding():
    grid = _e4m3_values()
    assert grid.max() == 448.0 and grid[1] == 2.0 ** -9
    # a tensor whose amax is exactly 448 has scale 1: codes are the values
    x = np.concatenate([grid, -grid, [448.0]]).astype(np.float32)
    t, s = W._to_storage(x, "fp8")
    assert s == 1.0
    assert np.array_equal(t.to(torch.float64).numpy(), x.astype(np.float64))
    # ties to even: 17 between 16 and 18 -> 16; 19 between 18 and 20 -> 20
    t, s = W._to_storage(np.array([448.0, 17.0, 19.0, 2.0 ** -10,
                                   3 * 2.0 ** -10], np.float32), "fp8")
    got = t.to(torch.float64).numpy()
    assert s == 1.0
    assert got[1] == 16.0 and got[2] == 20.0
    assert got[3] == 0.0                  # half of the smallest subnormal
    assert got[4] == 2.0 ** -8            # tie 1.5 ulp -> 2 ulp (even)


def test_e4m3_per_tensor_scale():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(4096).astype(np.float32)
    t, s = W._to_storage(x, "fp8")
    amax = float(np.abs(x).max())
    assert s == np.float32(amax / 448.0)
    deq = t.to(torch.float64).numpy() * s
    # largest magnitude maps to +/-448 (so nothing saturates) ...
    assert np.max(np.abs(t.to(torch.float64).numpy())) == 448.0
    # ... and every value is within half a step (relative 2^-4) of x,
    # or within half the smallest subnormal step for tiny values
    err = np.abs(deq - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) * 1.0001)


def test_prefill_inputs_deterministic_and_shaped():
    a = W.prefill_inputs(2, 4, 2, 5, 7, 16, dtype="bf16", causal=True, seed=3)
    b = W.prefill_inputs(2, 4, 2, 5, 7, 16, dtype="bf16", causal=True, seed=3)
    assert a.q.shape == (2, 4, 5, 16) and a.k.shape == (2, 2, 7, 16)
    assert a.q.dtype == torch.bfloat16 and a.causal
    assert torch.equal(a.q, b.q) and torch.equal(a.v, b.v)
    assert a.scale == 1.0 / 4.0
    f = W.prefill_inputs(1, 1, 1, 3, 3, 8, dtype="fp8")
    assert f.q.dtype == torch.float8_e4m3fn and len(f.descale) == 3


def test_decode_inputs_structure():
    lens = [1, 16, 17, 40, 0]
    di = W.decode_inputs(5, 4, 2, 8, page_size=16, lens=lens, seed=1,
                         max_pages=4, extra_pages=3)
    n = [1, 1, 2, 3, 0]
    assert di.k_pool.shape == (sum(n) + 3, 16, 2, 8)
    t = di.block_table.numpy()
    used = []
    for r in range(5):
        assert np.all(t[r, :n[r]] >= 0) and np.all(t[r, n[r]:] == -1)
        used += list(t[r, :n[r]])
    assert len(set(used)) == len(used)           # pages not shared
    # slots past the length of request 0 (length 1) are poisoned
    kp = di.k_pool.to(torch.float32).numpy()
    assert np.all(np.abs(kp[t[0, 0], 1:]) > 9000)
    assert np.all(np.abs(kp[t[0, 0], :1]) < 100)
    # request 1 fills its page exactly: no poison
    assert np.all(np.abs(kp[t[1, 0]]) < 100)
    assert di.seq_lens.dtype == torch.int32
    assert list(di.seq_lens.numpy()) == lens


@pytest.mark.parametrize("name", sorted(W.PREFILL_CONFIGS))
def test_config_table(name):
    c = W.PREFILL_CONFIGS[name]
    assert c["Hq"] % c["Hkv"] == 0 and c["d"] in (64, 128)


def test_decode_inputs_fp8_cache():
    bf = W.decode_inputs(3, 8, 2, 64, lens=[5, 33, 0], max_pages=4, seed=3)
    di = W.decode_inputs(3, 8, 2, 64, lens=[5, 33, 0], max_pages=4, seed=3,
                         kv_dtype="fp8")
    assert di.k_pool.dtype == torch.float8_e4m3fn
    assert di.v_pool.dtype == torch.float8_e4m3fn
    s_k, s_v = di.kv_descale
    assert s_k > 0 and s_v > 0
    # same draws, same tables and query as the bf16 cache
    assert torch.equal(di.block_table, bf.block_table)
    assert torch.equal(di.q, bf.q)
    # poison slots hold the largest finite code
    t = int(di.block_table[0, 0])
    assert torch.all(di.k_pool[t, 5:].float().abs() == W.E4M3_MAX)
    # real tokens: code * scale within e4m3 rounding of the drawn values
    k_real = di.k_pool[t, :5].float() * s_k
    assert torch.max(torch.abs(k_real - bf.k_pool[t, :5].float())) < 0.2
