"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: numbers
the pages print, closed forms, invariances, a different algorithm reaching
the same exact result (streaming softmax, tiled FA2), or brute force on tiny
inputs with a different softmax formula. A dropped term, a wrong sign or
index, or a transposed operand anywhere in ``oracle/`` fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------------------
# Worked example and labs of the capstone page
# ---------------------------------------------------------------------------
def test_worked_example_online_states():
    g = _load("online_softmax_worked_example.json")
    tol = 0.5 * 10 ** (-g["printed_decimals"])
    states = oracle.online_softmax_stats(g["blocks"])
    assert len(states) == 2
    for (m, l), want in zip(states, g["after_block"]):
        assert m == want["m"]
        assert abs(l - want["l"]) <= tol
    # the page's intermediate numbers of the second update
    m1, l1 = states[0]
    decay = math.exp(m1 - states[1][0])
    assert abs(decay - g["intermediates"]["decay_factor"]) <= tol
    assert abs(l1 * decay - g["intermediates"]["old_l_rescaled"]) <= tol


def test_worked_example_three_pass_equals_stream():
    g = _load("online_softmax_worked_example.json")
    flat = [x for b in g["blocks"] for x in b]
    m, l = oracle.softmax_stats(flat)
    want = g["after_block"][-1]
    assert m == want["m"]
    assert abs(l - want["l"]) <= 0.5e-3
    # closed form: e^-3 + e^-1 + e^-2 + e^0
    assert abs(l - (math.exp(-3) + math.exp(-1) + math.exp(-2) + 1.0)) < 1e-15


def test_lab2_vector_stream_vs_three_pass():
    """Block-wise softmax with one log-sum-exp combine over the blocks (the
    merge of [Capstone §2.2 step 4] applied to every block at once) reaches
    the oracle's P, for the lab's vector and block size."""
    g = _load("online_softmax_lab_vector.json")
    x, bs = g["vector"], g["block_size"]
    blocks = [x[i:i + bs] for i in range(0, len(x), bs)]
    # each block alone: its maximum and its exponentials against it
    loc = [(max(b), [math.exp(t - max(b)) for t in b]) for b in blocks]
    M = max(mb for mb, _ in loc)
    Z = sum(sum(e) * math.exp(mb - M) for mb, e in loc)
    combined = [ei * math.exp(mb - M) / Z for mb, e in loc for ei in e]
    p = oracle.safe_softmax(x)
    assert np.max(np.abs(p - np.array(combined))) <= g["max_abs_diff"] * 4
    assert abs(p.sum() - 1.0) < 1e-15
    # online_softmax_stats ends in the same (m, l)
    sm, sl = oracle.online_softmax_stats(blocks)[-1]
    assert sm == M
    assert abs(sl - Z) < 1e-14


def test_lab3_tiled_fa2_protocol():
    """Tiled attention in block log-sum-exp form vs the oracle, at the lab's
    seed, sizes and error bar. For each query tile and key block: the
    block's row maxima m_j, sums l_j and unnormalised product O_j =
    exp(S_j - m_j) V_j; then all blocks of the tile are combined at once
    with the merge identity of [Capstone §2.2 step 4] and appendix A Q1
    (weights exp(m_j - M)), dividing by l only at the end as in §4.2."""
    g = _load("tiled_fa2_lab_protocol.json")
    np.random.seed(g["legacy_numpy_seed"])
    N, d = g["seq_len"], g["head_dim"]
    Q = np.random.randn(N, d)
    K = np.random.randn(N, d)
    V = np.random.randn(N, d)
    scale = 1.0 / math.sqrt(d)
    Br, Bc = g["Br"], g["Bc"]
    out = np.zeros_like(Q)
    for i0 in range(0, N, Br):
        Qi = Q[i0:i0 + Br]
        ms, ls, os_ = [], [], []
        for j0 in range(0, N, Bc):
            s = scale * (Qi @ K[j0:j0 + Bc].T)
            mj = s.max(axis=1)
            e = np.exp(s - mj[:, None])
            ms.append(mj)
            ls.append(e.sum(axis=1))
            os_.append(e @ V[j0:j0 + Bc])
        ms, ls, os_ = np.stack(ms), np.stack(ls), np.stack(os_)
        w = np.exp(ms - ms.max(axis=0)[None])          # [blocks, rows]
        out[i0:i0 + Br] = ((w[..., None] * os_).sum(axis=0)
                           / (w * ls).sum(axis=0)[:, None])
    o, lse = oracle.attention(Q[None, None], K[None, None], V[None, None],
                              scale)
    assert np.max(np.abs(o[0, 0] - out)) < g["pass_if_max_abs_error_below"]


# ---------------------------------------------------------------------------
# Brute force with a different softmax formula (no max subtraction)
# ---------------------------------------------------------------------------
def _brute(q, k, v, scale, causal):
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    O = np.zeros((B, Hq, Nq, d))
    L = np.full((B, Hq, Nq), -math.inf)
    for b in range(B):
        for h in range(Hq):
            for i in range(Nq):
                w = []
                for j in range(Nk):
                    if causal and j > i + Nk - Nq:
                        continue
                    s = scale * sum(float(q[b, h, i, t]) * float(k[b, h // g, j, t])
                                    for t in range(d))
                    w.append((j, math.exp(s)))
                z = sum(e for _, e in w)
                if z == 0.0:
                    continue
                L[b, h, i] = math.log(z)
                for t in range(d):
                    O[b, h, i, t] = sum(e * float(v[b, h // g, j, t])
                                        for j, e in w) / z
    return O, L


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1, 1), (1, 2, 1, 3, 3, 2),
                                   (2, 4, 2, 4, 3, 3), (1, 2, 2, 2, 4, 3),
                                   (1, 3, 1, 4, 2, 1)])
def test_brute_force_tiny(shape, causal):
    B, Hq, Hkv, Nq, Nk, d = shape
    rng = np.random.default_rng(7)
    q = _rand(rng, B, Hq, Nq, d)
    k = _rand(rng, B, Hkv, Nk, d)
    v = _rand(rng, B, Hkv, Nk, d)
    scale = 0.7
    o, lse = oracle.attention(q, k, v, scale, causal=causal)
    bo, bl = _brute(q, k, v, scale, causal)
    assert np.max(np.abs(o - bo)) < 1e-14
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - bl[fin]), initial=0.0) < 1e-13


# ---------------------------------------------------------------------------
# Closed forms and invariances
# ---------------------------------------------------------------------------
def test_rows_of_p_sum_to_one():
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 1, 2, 9, 5), _rand(rng, 1, 2, 13, 5), _rand(rng, 1, 2, 13, 5)
    scale = 0.4
    for causal in (False, True):
        _, lse = oracle.attention(q, k, v, scale, causal=causal)
        S = scale * np.einsum("bhid,bhjd->bhij", q, k)
        if causal:
            i = np.arange(9)[:, None]
            j = np.arange(13)[None, :]
            S = np.where(j <= i + 4, S, -np.inf)
        tot = np.exp(S - lse[..., None]).sum(-1)
        assert np.max(np.abs(tot - 1.0)) < 1e-13


def test_constant_scores_give_mean_of_v():
    rng = np.random.default_rng(2)
    Nk, d = 37, 6
    q = np.zeros((1, 1, 5, d))
    k, v = _rand(rng, 1, 1, Nk, d), _rand(rng, 1, 1, Nk, d)
    o, lse = oracle.attention(q, k, v, 0.3)
    assert np.max(np.abs(o[0, 0] - v[0, 0].mean(0)[None])) < 1e-14
    assert np.max(np.abs(lse - math.log(Nk))) < 1e-14
    # all key rows equal: uniform weights again, LSE shifted by the score
    q = _rand(rng, 1, 1, 4, d)
    k = np.repeat(_rand(rng, 1, 1, 1, d), Nk, axis=2)
    o, lse = oracle.attention(q, k, v, 0.3)
    assert np.max(np.abs(o[0, 0] - v[0, 0].mean(0)[None])) < 1e-14
    want = 0.3 * (q[0, 0] @ k[0, 0, 0]) + math.log(Nk)
    assert np.max(np.abs(lse[0, 0] - want)) < 1e-13


def test_single_key():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 2, 2, 6, 4), _rand(rng, 2, 2, 1, 4), _rand(rng, 2, 2, 1, 4)
    o, lse = oracle.attention(q, k, v, 1.3)
    assert np.max(np.abs(o - v)) < 1e-15
    assert np.max(np.abs(lse - 1.3 * np.einsum("bhid,bhjd->bhi", q, k))) < 1e-13


def test_causal_row_zero_is_v0():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 1, 3, 11, 8), _rand(rng, 1, 3, 11, 8), _rand(rng, 1, 3, 11, 8)
    o, lse = oracle.attention(q, k, v, 0.35, causal=True)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    assert np.max(np.abs(lse[:, :, 0] - 0.35 * np.sum(q[:, :, 0] * k[:, :, 0], -1))) < 1e-14
    # the last row sees every key: equals the non-causal last row
    on, ln = oracle.attention(q, k, v, 0.35, causal=False)
    assert np.max(np.abs(o[:, :, -1] - on[:, :, -1])) < 1e-14
    assert np.max(np.abs(lse[:, :, -1] - ln[:, :, -1])) < 1e-14


def test_causal_bottom_right_alignment():
    rng = np.random.default_rng(5)
    # Nq < Nk: row i sees keys 0..i+Nk-Nq
    q, k, v = _rand(rng, 1, 1, 3, 4), _rand(rng, 1, 1, 7, 4), _rand(rng, 1, 1, 7, 4)
    o, lse = oracle.attention(q, k, v, 0.5, causal=True)
    for i in range(3):
        oi, li = oracle.attention(q[:, :, i:i + 1], k[:, :, :i + 5],
                                  v[:, :, :i + 5], 0.5)
        assert np.max(np.abs(o[:, :, i] - oi[:, :, 0])) < 1e-14
        assert abs(lse[0, 0, i] - li[0, 0, 0]) < 1e-14
    # Nq > Nk: the first Nq-Nk rows see nothing -> O = 0, LSE = -inf
    q = _rand(rng, 1, 1, 6, 4)
    o, lse = oracle.attention(q, k[:, :, :2], v[:, :, :2], 0.5, causal=True)
    assert np.all(o[0, 0, :4] == 0.0) and np.all(np.isneginf(lse[0, 0, :4]))
    assert np.all(np.isfinite(lse[0, 0, 4:]))
    assert np.array_equal(o[0, 0, 4], v[0, 0, 0])
    assert not np.any(np.isnan(o))


def test_no_keys():
    q = np.ones((1, 1, 3, 2))
    k = np.ones((1, 1, 0, 2))
    o, lse = oracle.attention(q, k, k, 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_key_permutation_invariance():
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 2, 2, 7, 5), _rand(rng, 2, 2, 19, 5), _rand(rng, 2, 2, 19, 5)
    perm = rng.permutation(19)
    o1, l1 = oracle.attention(q, k, v, 0.6)
    o2, l2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.6)
    assert np.max(np.abs(o1 - o2)) < 1e-14 and np.max(np.abs(l1 - l2)) < 1e-13
    # but a permutation of V alone changes O (operands are not confused)
    o3, _ = oracle.attention(q, k, v[:, :, perm], 0.6)
    assert np.max(np.abs(o1 - o3)) > 1e-3


def test_key_shift_invariance():
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 1, 2, 6, 5), _rand(rng, 1, 2, 9, 5), _rand(rng, 1, 2, 9, 5)
    u = _rand(rng, 5)
    o1, l1 = oracle.attention(q, k, v, 0.45)
    o2, l2 = oracle.attention(q, k + u, v, 0.45)
    assert np.max(np.abs(o1 - o2)) < 1e-13
    assert np.max(np.abs(l2 - (l1 + 0.45 * q @ u))) < 1e-13


def test_linearity_in_v():
    rng = np.random.default_rng(9)
    q, k = _rand(rng, 1, 2, 6, 5), _rand(rng, 1, 2, 9, 5)
    v1, v2 = _rand(rng, 1, 2, 9, 5), _rand(rng, 1, 2, 9, 5)
    a, b = 1.7, -0.3
    o1, _ = oracle.attention(q, k, v1, 0.5)
    o2, _ = oracle.attention(q, k, v2, 0.5)
    o3, _ = oracle.attention(q, k, a * v1 + b * v2, 0.5)
    assert np.max(np.abs(o3 - (a * o1 + b * o2))) < 1e-13


def test_scale_multiplies_scores():
    rng = np.random.default_rng(10)
    q, k, v = _rand(rng, 1, 1, 5, 4), _rand(rng, 1, 1, 8, 4), _rand(rng, 1, 1, 8, 4)
    o1, l1 = oracle.attention(q, k, v, 0.5)
    o2, l2 = oracle.attention(2.0 * q, k, v, 0.25)
    assert np.max(np.abs(o1 - o2)) < 1e-14 and np.max(np.abs(l1 - l2)) < 1e-14


def test_gqa_equals_repeated_heads():
    rng = np.random.default_rng(11)
    Hq, Hkv = 8, 2
    q = _rand(rng, 2, Hq, 5, 4)
    k, v = _rand(rng, 2, Hkv, 7, 4), _rand(rng, 2, Hkv, 7, 4)
    o, lse = oracle.attention(q, k, v, 0.5, causal=True)
    kr = np.repeat(k, Hq // Hkv, axis=1)      # head h -> kv head h // 4
    vr = np.repeat(v, Hq // Hkv, axis=1)
    o2, l2 = oracle.attention(q, kr, vr, 0.5, causal=True)
    assert np.max(np.abs(o - o2)) < 1e-15 and np.max(np.abs(lse - l2)) < 1e-15
    # and each query head matches a one-head call on its own kv head
    for h in range(Hq):
        oh, lh = oracle.attention(q[:, h:h + 1], k[:, h // 4:h // 4 + 1],
                                  v[:, h // 4:h // 4 + 1], 0.5, causal=True)
        assert np.max(np.abs(o[:, h:h + 1] - oh)) < 1e-15


def test_row_subset_matches_full():
    rng = np.random.default_rng(12)
    q, k, v = _rand(rng, 1, 2, 20, 4), _rand(rng, 1, 1, 20, 4), _rand(rng, 1, 1, 20, 4)
    rows = np.array([0, 3, 19, 7])
    for causal in (False, True):
        of, lf = oracle.attention(q, k, v, 0.5, causal=causal)
        os_, ls = oracle.attention(q, k, v, 0.5, causal=causal, rows=rows)
        assert np.array_equal(os_, of[:, :, rows])
        assert np.array_equal(ls, lf[:, :, rows])


# ---------------------------------------------------------------------------
# Merge of partials (split-KV)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cuts", [(0, 13, 40), (0, 1, 2, 40), (0, 20, 20, 40),
                                  (0, 39, 40), (0, 10, 17, 31, 40)])
def test_merge_identity(cuts):
    rng = np.random.default_rng(13)
    q, k, v = _rand(rng, 1, 3, 4, 6), _rand(rng, 1, 3, 40, 6), _rand(rng, 1, 3, 40, 6)
    o_full, l_full = oracle.attention(q, k, v, 0.5)
    parts_o, parts_l = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = oracle.attention(q, k[:, :, a:b], v[:, :, a:b], 0.5)
        parts_o.append(o)
        parts_l.append(l)
    o, l = oracle.merge_partials(np.stack(parts_o), np.stack(parts_l))
    assert np.max(np.abs(o - o_full)) < 1e-13
    assert np.max(np.abs(l - l_full)) < 1e-13


def test_merge_two_blocks_page_form():
    """The page's unnormalised form: O_new = diag(l_A e^{m_A-m}/l) O_A +
    diag(e^{m_B-m}/l) (P_B V_B), with O_A normalised and P_B V_B not."""
    rng = np.random.default_rng(14)
    x = rng.standard_normal(12) * 3
    V = rng.standard_normal((12, 3))
    A, B = slice(0, 5), slice(5, 12)
    mA, lA = oracle.softmax_stats(x[A])
    mB, lB = oracle.softmax_stats(x[B])
    OA = (np.exp(x[A] - mA) / lA) @ V[A]
    PBVB = np.exp(x[B] - mB) @ V[B]
    m = max(mA, mB)
    lnew = lA * math.exp(mA - m) + lB * math.exp(mB - m)
    Onew = (lA * math.exp(mA - m) / lnew) * OA + (math.exp(mB - m) / lnew) * PBVB
    o, L = oracle.merge_partials(np.stack([OA, PBVB / lB]),
                                 np.array([mA + math.log(lA), mB + math.log(lB)]))
    assert np.max(np.abs(o - Onew)) < 1e-14
    assert abs(L - (m + math.log(lnew))) < 1e-14
    assert np.max(np.abs(Onew - oracle.safe_softmax(x) @ V)) < 1e-14


def test_merge_all_empty():
    o, l = oracle.merge_partials(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(o == 0) and np.all(np.isneginf(l))


# ---------------------------------------------------------------------------
# Paged decode
# ---------------------------------------------------------------------------
def _tiny_pages(rng, lens, page, Hkv, d, perm_seed):
    n = [-(-L // page) for L in lens]
    total = sum(n)
    kp = rng.standard_normal((total, page, Hkv, d))
    vp = rng.standard_normal((total, page, Hkv, d))
    perm = np.random.default_rng(perm_seed).permutation(total)
    table = np.full((len(lens), max(n + [1])), -1, dtype=np.int64)
    s = 0
    for r, c in enumerate(n):
        table[r, :c] = perm[s:s + c]
        s += c
    return kp, vp, table


def test_paged_decode_equals_contiguous():
    rng = np.random.default_rng(15)
    lens, page, Hq, Hkv, d = [1, 4, 5, 11, 16, 17], 4, 6, 2, 3
    kp, vp, table = _tiny_pages(rng, lens, page, Hkv, d, 0)
    q = rng.standard_normal((len(lens), Hq, d))
    o, lse = oracle.paged_decode(q, kp, vp, table, lens, page, 0.8)
    for r, L in enumerate(lens):
        # contiguous cache rebuilt token by token
        K = np.zeros((Hkv, L, d))
        V = np.zeros((Hkv, L, d))
        for t in range(L):
            K[:, t] = kp[table[r, t // page], t % page]
            V[:, t] = vp[table[r, t // page], t % page]
        oc, lc = oracle.attention(q[r][None, :, None], K[None], V[None], 0.8)
        assert np.max(np.abs(o[r] - oc[0, :, 0])) < 1e-15
        assert np.max(np.abs(lse[r] - lc[0, :, 0])) < 1e-15


def test_paged_decode_relabel_and_poison():
    rng = np.random.default_rng(16)
    lens, page, Hq, Hkv, d = [3, 9, 12], 4, 4, 2, 5
    kp, vp, table = _tiny_pages(rng, lens, page, Hkv, d, 1)
    q = rng.standard_normal((3, Hq, d))
    o1, l1 = oracle.paged_decode(q, kp, vp, table, lens, page, 0.5)
    # move every page to a new physical slot
    perm = np.random.default_rng(99).permutation(kp.shape[0])
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1)
    o2, l2 = oracle.paged_decode(q, kp2, vp2, table2, lens, page, 0.5)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # poisoning the slots past each length changes nothing
    for r, L in enumerate(lens):
        last = table[r, (L - 1) // page]
        kp[last, L - ((L - 1) // page) * page:] = 1e4
        vp[last, L - ((L - 1) // page) * page:] = -1e4
    o3, l3 = oracle.paged_decode(q, kp, vp, table, lens, page, 0.5)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


def test_paged_decode_group_and_empty():
    rng = np.random.default_rng(17)
    lens, page, Hq, Hkv, d = [0, 2, 7], 4, 4, 2, 3
    kp, vp, table = _tiny_pages(rng, lens, page, Hkv, d, 2)
    q = rng.standard_normal((3, Hq, d))
    o, lse = oracle.paged_decode(q, kp, vp, table, lens, page, 0.5)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    # request 1 has two tokens in page table[1,0]: brute force per head
    for h in range(Hq):
        kv = h // 2
        ks = kp[table[1, 0], :2, kv]
        vs = vp[table[1, 0], :2, kv]
        s = 0.5 * (ks @ q[1, h])
        w = np.exp(s) / np.exp(s).sum()
        assert np.max(np.abs(o[1, h] - w @ vs)) < 1e-15
        assert abs(lse[1, h] - math.log(np.exp(s).sum())) < 1e-14


# ---------------------------------------------------------------------------
# fp8 (per-tensor scaled codes)
# ---------------------------------------------------------------------------
def test_fp8_dequantisation_and_scales():
    rng = np.random.default_rng(18)
    # code values drawn from a few exact e4m3 numbers
    vals = np.array([-448, -3.5, -1, -0.0625, 0, 0.125, 1.5, 2, 96, 448.0])
    qc = rng.choice(vals, (1, 2, 5, 4))
    kc = rng.choice(vals, (1, 2, 7, 4))
    vc = rng.choice(vals, (1, 2, 7, 4))
    sq, sk, sv = 0.003, 0.0021, 0.0117
    o, lse = oracle.attention_fp8(qc, kc, vc, sq, sk, sv, 0.5)
    o2, l2 = oracle.attention(qc * sq, kc * sk, vc * sv, 0.5)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)
    # only s_q * s_k matters for the scores; O is linear in s_v
    o3, l3 = oracle.attention_fp8(qc, kc, vc, sk, sq, 2 * sv, 0.5)
    assert np.max(np.abs(o3 - 2 * o)) < 1e-13
    assert np.max(np.abs(l3 - lse)) < 1e-13
    o4, l4 = oracle.attention_fp8(qc, kc, vc, 1.0, sq * sk, sv, 0.5)
    assert np.max(np.abs(o4 - o)) < 1e-13


def test_paged_decode_fp8_cache_scales():
    # an e4m3 cache: codes times one scale per pool; the decode of those
    # values is the plain paged decode of the dequantised pools, only
    # scale * s_k matters for the scores and O is linear in s_v
    rng = np.random.default_rng(19)
    vals = np.array([-448, -7.5, -1, -0.125, 0, 0.25, 1.75, 3, 64, 448.0])
    n_pages, page, Hkv, d = 6, 4, 2, 3
    kc = rng.choice(vals, (n_pages, page, Hkv, d))
    vc = rng.choice(vals, (n_pages, page, Hkv, d))
    q = rng.standard_normal((2, 4, d))
    table = np.array([[3, 0, 5], [1, 4, -1]])
    lens = np.array([10, 6])
    sk, sv = 0.0031, 0.0087
    o, lse = oracle.paged_decode_fp8(q, kc, vc, sk, sv, table, lens, page, 0.6)
    # the dequantised pools by hand, gathered request by request
    for r in range(2):
        n = -(-lens[r] // page)
        K = np.concatenate([kc[table[r, p]] for p in range(n)])[: lens[r]] * sk
        V = np.concatenate([vc[table[r, p]] for p in range(n)])[: lens[r]] * sv
        for h in range(4):
            hk = h // 2
            sc = 0.6 * (K[:, hk, :] @ q[r, h])
            w = np.exp(sc - sc.max())
            assert abs(np.log(w.sum()) + sc.max() - lse[r, h]) < 1e-12
            assert np.max(np.abs((w / w.sum()) @ V[:, hk, :] - o[r, h])) < 1e-12
    o2, l2 = oracle.paged_decode_fp8(q, kc, vc, 1.0, 2 * sv, table, lens,
                                     page, 0.6 * sk)
    assert np.max(np.abs(o2 - 2 * o)) < 1e-12
    assert np.max(np.abs(l2 - lse)) < 1e-12


def test_paged_prefill_rows_are_decodes_of_prefixes():
    # causal chunked prefill: query i of the chunk is the token at position
    # L - Nq + i, so it is the decode of the request's first L - Nq + i + 1
    # cached tokens (an independent route: paged_decode with shorter lengths)
    import workloads as W
    di = W.paged_prefill_inputs(3, 4, 2, 8, 5, lens=[40, 5, 17], max_pages=4,
                                seed=12)
    q = W.as_f64(di.q)
    kp, vp = W.as_f64(di.k_pool), W.as_f64(di.v_pool)
    bt, sl = di.block_table.numpy(), di.seq_lens.numpy()
    o, lse = oracle.paged_prefill(q, kp, vp, bt, sl, 16, 0.3, causal=True)
    for i in range(5):
        lens_i = np.maximum(sl - 5 + i + 1, 0)
        od, ld = oracle.paged_decode(q[:, :, i], kp, vp, bt, lens_i, 16, 0.3)
        assert np.max(np.abs(od - o[:, :, i])) < 1e-12
        live = np.isfinite(ld)
        assert np.array_equal(live, np.isfinite(lse[:, :, i]))
        assert np.max(np.abs(ld[live] - lse[:, :, i][live])) < 1e-12
    # non-causal: every query of a request sees all of its L tokens, the
    # same as a decode of each query against the full cache
    o2, _ = oracle.paged_prefill(q, kp, vp, bt, sl, 16, 0.3, causal=False)
    for i in range(5):
        od, _ = oracle.paged_decode(q[:, :, i], kp, vp, bt, sl, 16, 0.3)
        assert np.max(np.abs(od - o2[:, :, i])) < 1e-12


# ---------------------------------------------------------------- backward
# The gradient of the definition is pinned by numerical differentiation of
# the forward oracle (central differences in fp64 on tiny inputs, an
# independent route to the same derivative) and by invariants of the
# softmax that a dropped term, a wrong sign or a transposed operand breaks.
def _loss_grad_fd(q, k, v, g, scale, causal, eps=1e-6):
    """Central-difference gradients of L = sum(O * g) w.r.t. q, k, v."""
    def loss(q_, k_, v_):
        o, _ = oracle.attention(q_, k_, v_, scale, causal=causal)
        return float(np.sum(o * g))
    out = []
    for x in (q, k, v):
        gx = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[i] += eps
            xm[i] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            idx = [q is x, k is x, v is x].index(True)
            args_p[idx], args_m[idx] = xp, xm
            gx[i] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        out.append(gx)
    return out


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal", [
    (1, 1, 1, 4, 5, 3, False),
    (1, 2, 1, 5, 5, 3, True),      # GQA, causal square
    (2, 2, 2, 3, 6, 2, True),      # causal, Nk > Nq (bottom-right)
    (1, 1, 1, 6, 3, 2, True),      # causal, Nq > Nk: rows 0..2 see no key
])
def test_backward_matches_finite_differences(B, Hq, Hkv, Nq, Nk, d, causal):
    rng = np.random.default_rng(7 + Nq * Nk)
    q = rng.standard_normal((B, Hq, Nq, d))
    k = rng.standard_normal((B, Hkv, Nk, d))
    v = rng.standard_normal((B, Hkv, Nk, d))
    g = rng.standard_normal((B, Hq, Nq, d))
    scale = 0.7
    dq, dk, dv = oracle.attention_backward(q, k, v, g, scale, causal=causal)
    fq, fk, fv = _loss_grad_fd(q, k, v, g, scale, causal)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        assert np.max(np.abs(a - b)) < 1e-7


def test_backward_key_shift_gives_zero_key_gradient_sum():
    # adding u to every key adds scale*q_i.u to every visible score of row i:
    # the softmax is unchanged, so sum_j dK_j = 0 (for every KV head)
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 4, 33, 8))
    k = rng.standard_normal((2, 2, 40, 8))
    v = rng.standard_normal((2, 2, 40, 8))
    g = rng.standard_normal((2, 4, 33, 8))
    for causal in (False, True):
        _, dk, _ = oracle.attention_backward(q, k, v, g, 0.3, causal=causal)
        assert np.max(np.abs(dk.sum(axis=2))) < 1e-12


def test_backward_equal_keys_give_zero_dq():
    # all keys equal: every score of a row is the same, P is uniform
    # whatever Q is, so dQ = 0 (and dV_j = mean over rows of dO)
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 7, 5))
    k = np.repeat(rng.standard_normal((1, 1, 1, 5)), 9, axis=2)
    v = rng.standard_normal((1, 1, 9, 5))
    g = rng.standard_normal((1, 1, 7, 5))
    dq, _, dv = oracle.attention_backward(q, k, v, g, 0.5)
    assert np.max(np.abs(dq)) < 1e-12
    want = np.repeat(g.sum(axis=2, keepdims=True) / 9, 9, axis=2)
    assert np.max(np.abs(dv - want)) < 1e-12


def test_backward_scale_placement():
    # f(Q; s) = f(s Q; 1): dQ at scale s is s times dQ at scale 1 taken at
    # s Q, and dK at scale s equals dK at scale 1 taken at s Q
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 2, 6, 4))
    k = rng.standard_normal((1, 2, 8, 4))
    v = rng.standard_normal((1, 2, 8, 4))
    g = rng.standard_normal((1, 2, 6, 4))
    s = 0.37
    dq_s, dk_s, dv_s = oracle.attention_backward(q, k, v, g, s, causal=True)
    dq_1, dk_1, dv_1 = oracle.attention_backward(s * q, k, v, g, 1.0,
                                                 causal=True)
    assert np.max(np.abs(dq_s - s * dq_1)) < 1e-12
    assert np.max(np.abs(dk_s - dk_1)) < 1e-12
    assert np.max(np.abs(dv_s - dv_1)) < 1e-12


def test_backward_gqa_is_sum_over_repeated_heads():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 6, 5, 3))
    k = rng.standard_normal((1, 2, 7, 3))
    v = rng.standard_normal((1, 2, 7, 3))
    g = rng.standard_normal((1, 6, 5, 3))
    dq, dk, dv = oracle.attention_backward(q, k, v, g, 0.9, causal=True)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    dq2, dk2, dv2 = oracle.attention_backward(q, kr, vr, g, 0.9, causal=True)
    assert np.max(np.abs(dq - dq2)) < 1e-12
    assert np.max(np.abs(dk - dk2.reshape(1, 2, 3, 7, 3).sum(axis=2))) < 1e-12
    assert np.max(np.abs(dv - dv2.reshape(1, 2, 3, 7, 3).sum(axis=2))) < 1e-12


def test_backward_linear_in_upstream_gradient():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 1, 6, 4))
    k = rng.standard_normal((1, 1, 6, 4))
    v = rng.standard_normal((1, 1, 6, 4))
    g1 = rng.standard_normal((1, 1, 6, 4))
    g2 = rng.standard_normal((1, 1, 6, 4))
    a = oracle.attention_backward(q, k, v, g1, 0.5)
    b = oracle.attention_backward(q, k, v, g2, 0.5)
    c = oracle.attention_backward(q, k, v, 2.0 * g1 - 3.0 * g2, 0.5)
    for x, y, z in zip(a, b, c):
        assert np.max(np.abs(z - (2.0 * x - 3.0 * y))) < 1e-12


def test_backward_rows_without_keys_have_zero_gradient():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 1, 6, 3))
    k = rng.standard_normal((1, 1, 3, 3))
    v = rng.standard_normal((1, 1, 3, 3))
    g = rng.standard_normal((1, 1, 6, 3))
    dq, _, _ = oracle.attention_backward(q, k, v, g, 1.0, causal=True)
    assert np.all(dq[0, 0, :3] == 0) and np.any(dq[0, 0, 3:] != 0)


# ---------------------------------------------------------------------------
# Report-only fp8 diagnostic: P rounded to e4m3
# ---------------------------------------------------------------------------
def test_round_e4m3_matches_torch_cast():
    """round_e4m3 equals torch's float8_e4m3fn conversion (a library
    routine) on fp32 values: normals, subnormals, exact ties, the largest
    finite value and zero."""
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0,
        rng.uniform(-2 ** -6, 2 ** -6, 5000),            # subnormal range
        np.array([0.0, 448.0, -448.0, 2 ** -9, 3 * 2 ** -10, 1.0625,
                  1.1875, 240.0, 440.0, 0.01171875]),
    ]).astype(np.float32)
    x = x[np.abs(x) <= 448.0]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_e4m3(x.astype(np.float64)), want)


def test_p_e4m3_diagnostic_special_cases():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 2, 20, 16))
    k = rng.standard_normal((1, 1, 30, 16))
    v = rng.standard_normal((1, 1, 30, 16))
    # weights that are a convex combination: V of all ones gives O = 1
    o, _ = oracle.attention_fp8_p_e4m3(q, k, np.ones_like(v), 1.0, 1.0, 1.0,
                                       0.3)
    assert np.max(np.abs(o - 1.0)) < 1e-14
    # scores whose exponentials are powers of two are not rounded at all:
    # then the diagnostic equals the oracle
    kk = np.zeros((1, 1, 4, 16))
    kk[0, 0, :, 0] = [0.0, -1.0, -2.0, -3.0]
    qq = np.zeros((1, 1, 3, 16))
    qq[0, 0, :, 0] = math.log(2.0)
    vv = rng.standard_normal((1, 1, 4, 16))
    o1, l1 = oracle.attention_fp8_p_e4m3(qq, kk, vv, 1.0, 1.0, 1.0, 1.0)
    o2, l2 = oracle.attention(qq, kk, vv, 1.0)
    assert np.max(np.abs(o1 - o2)) < 1e-14 and np.array_equal(l1, l2)
    # causal row 0 sees one key: O = V[0]
    o3, _ = oracle.attention_fp8_p_e4m3(q[:, :1], k[:, :, :20], v[:, :, :20],
                                        1.0, 1.0, 1.0, 0.25, causal=True)
    assert np.max(np.abs(o3[0, 0, 0] - v[0, 0, 0])) < 1e-14
    # and the rounding moves O by no more than the e4m3 step allows
    o4, _ = oracle.attention_fp8_p_e4m3(q, k, v, 1.0, 1.0, 1.0, 0.25)
    o5, _ = oracle.attention(q, k, v, 0.25)
    bound = 2 * 2 ** -4 * np.max(np.abs(v))
    assert 0 < np.max(np.abs(o4 - o5)) <= bound
