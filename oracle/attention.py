"""Plain, slow, fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library and imports nothing from it.

Sources (cited by page and section; no code is taken from them):

* [FA3-guide]   "Flash Attention 3 指南：GPU IO 优化的终极武器"
                (guijiagi.com, flash-attention-3-guide). No headings; cited by
                the name of the listing, e.g. the ``flash_attn_v3_fp8`` listing.
* [FA3-paged]   "FlashAttention V3 实战：Hopper 架构下的 Paged KV Cache 协同优化"
                (ybb.press, gpu-parallel 14727). Sections 一 (problem), 3.1
                (online softmax and tiling), 3.2 (paged KV cache).
* [Capstone]    "项目三：榨干片上 SRAM——CUDA Softmax 与 Attention 算子极致性能调优"
                (lilinji.mintlify.site capstone). Sections 1.1, 2.1, 2.2
                (steps 1-5), 4.1, 4.2, lab 3, 7.3, appendix A (Q1).

What is computed is the plain definition of scaled dot-product attention,
O = softmax(scale * Q K^T) V, written out with the score matrix S
materialised and the three-pass safe softmax of [Capstone §2.1]. Attention
is exact: the streaming (online-softmax) algorithm the GPU runs reaches the
same result up to rounding order ([Capstone §2.2 step 5], appendix A Q1), so
the oracle does not follow the tiled algorithm at all.

Readings taken where the pages are silent (each is also listed in the design
notes of the repository):

* LSE is the natural-log log-sum-exp of the *scaled* scores of a row,
  LSE_i = m_i + ln(l_i). The pages keep (m, l) per row [Capstone §6.1, the
  row about not writing P to HBM]; LSE is that pair folded into one number.
* Causal masking is bottom-right aligned: key j is visible to query i iff
  j <= i + (Nk - Nq). For Nq == Nk this is the lower triangle of
  [Capstone §7.3, question 2]; for a single decode query it sees all keys.
* Grouped-query attention: query head h reads KV head h // (Hq // Hkv).
* A row whose keys are all masked has l = 0 (an empty sum): its O is 0 and
  its LSE is -inf (never NaN).
* FP8: values are e4m3 codes times a per-tensor fp32 scale; the oracle
  multiplies them out in fp64 (exact) and does NOT model the kernel's
  re-quantisation of P ([FA3-guide] ``flash_attn_v3_fp8`` listing).

Backward: the pages say only that the backward pass re-computes P on chip
from Q, K and the saved row statistics instead of reading a stored P
([Capstone §6.1], the row about writing P to HBM; §7.3 question 1). What it
must produce is the gradient of the definition, which the oracle writes out
with the chain rule through the materialised softmax (see
``attention_backward``).

Pins: every function here is checked by ``tests/test_oracle_pins.py``
against values the pages print, closed forms, invariants and brute force.
The fp8 path's re-quantisation error of P is the one part left unpinned
("parity unpinned": bounded only by the tolerance).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "softmax_stats",
    "online_softmax_stats",
    "safe_softmax",
    "attention",
    "attention_fp8",
    "round_e4m3",
    "attention_fp8_p_e4m3",
    "merge_partials",
    "gather_paged_kv",
    "paged_decode",
    "paged_decode_fp8",
    "paged_prefill",
    "attention_backward",
]


# --------------------------------------------------------------------------
# Softmax building blocks
# --------------------------------------------------------------------------
def softmax_stats(x):
    """Three-pass safe softmax statistics of a 1-D vector [Capstone §2.1].

    Pass 1: m = max_j x_j.  Pass 2: l = sum_j exp(x_j - m).
    Returns (m, l) as Python floats. An all -inf vector gives (-inf, 0).
    """
    x = np.asarray(x, dtype=np.float64)
    m = float(np.max(x))
    if m == -math.inf:
        return m, 0.0
    return m, float(np.sum(np.exp(x - m)))


def safe_softmax(x):
    """Pass 3 of [Capstone §2.1]: P_i = exp(x_i - m) / l."""
    x = np.asarray(x, dtype=np.float64)
    m, l = softmax_stats(x)
    if l == 0.0:
        return np.zeros_like(x)
    return np.exp(x - m) / l


def online_softmax_stats(blocks):
    """Streaming (m, l) over a sequence of blocks [Capstone §2.2 steps 3-4].

    Each block's own statistics (m_B, l_B) come from the three-pass
    ``softmax_stats``; they are folded into the running pair with the
    two-block merge of step 4: m = max(m_run, m_B) and
    l = l_run * exp(m_run - m) + l_B * exp(m_B - m). A side that has seen no
    finite value (m = -inf, l = 0) adds nothing to the sum. Returns the list
    of (m, l) after each block, so a test can compare every intermediate
    state with the page's worked example.
    """
    def weight(mx, m):
        return 0.0 if mx == -math.inf else math.exp(mx - m)

    m_run, l_run = -math.inf, 0.0
    states = []
    for blk in blocks:
        m_b, l_b = softmax_stats(blk)
        m = max(m_run, m_b)
        if m > -math.inf:
            l_run = l_run * weight(m_run, m) + l_b * weight(m_b, m)
            m_run = m
        states.append((m_run, l_run))
    return states


# --------------------------------------------------------------------------
# Attention forward (the definition)
# --------------------------------------------------------------------------
def _visible(rows, nq, nk):
    """Boolean [len(rows), nk]: key j visible to query row i (bottom-right)."""
    rows = np.asarray(rows, dtype=np.int64)
    return np.arange(nk, dtype=np.int64)[None, :] <= (rows[:, None] + (nk - nq))


def attention(q, k, v, scale, causal=False, rows=None):
    """Exact attention, fp64, one (batch, query-head) at a time.

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d] (any real dtype, used as fp64).
    scale: the multiplier applied to Q K^T before the softmax
    ([Capstone §1.1] uses 1/sqrt(d); the caller passes it).
    causal: bottom-right aligned lower-triangular mask.
    rows: optional 1-D array of query-row indices; only those rows are
    computed (each output row depends on its own query only, so any subset
    is the same definition evaluated at fewer points).

    Returns (O, LSE): O [B, Hq, R, d] fp64 and LSE [B, Hq, R] fp64, with
    R = Nq, or len(rows) when rows is given.

    Steps per (b, h): S = scale * Q K^T (materialised) -> mask -> three-pass
    softmax (m, l, P) [Capstone §2.1] -> O = P V, LSE = m + ln l.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k and v")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    if rows is None:
        rows = np.arange(Nq, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]

    out = np.zeros((B, Hq, R, d), dtype=np.float64)
    lse = np.full((B, Hq, R), -np.inf, dtype=np.float64)
    if R == 0 or Nk == 0:
        return out, lse
    vis = _visible(rows, Nq, Nk) if causal else None
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            S = scale * (q[b, h, rows, :] @ k[b, hk].T)        # [R, Nk]
            if vis is not None:
                S = np.where(vis, S, -np.inf)
            m = np.max(S, axis=1)                               # pass 1
            live = m > -np.inf
            E = np.zeros_like(S)
            E[live] = np.exp(S[live] - m[live, None])           # pass 2
            l = np.sum(E, axis=1)
            P = np.zeros_like(S)
            P[live] = E[live] / l[live, None]                   # pass 3
            out[b, h] = P @ v[b, hk]
            lse[b, h, live] = m[live] + np.log(l[live])
    return out, lse


def attention_fp8(qc, kc, vc, s_q, s_k, s_v, scale, causal=False, rows=None):
    """Attention on per-tensor scaled e4m3 inputs [FA3-guide, fp8 listing].

    qc, kc, vc hold the *values* of the e4m3 codes (as any real dtype);
    s_q, s_k, s_v are the per-tensor scales, so the real inputs are
    X = code * s_X. The products are exact in fp64 (a 4-bit significand
    times a 24-bit one), after which this is ``attention`` on X.
    P's re-quantisation inside the kernel is not modelled.
    """
    qx = np.asarray(qc, dtype=np.float64) * float(s_q)
    kx = np.asarray(kc, dtype=np.float64) * float(s_k)
    vx = np.asarray(vc, dtype=np.float64) * float(s_v)
    return attention(qx, kx, vx, scale, causal=causal, rows=rows)


def round_e4m3(x):
    """Round fp64 values to the nearest OCP e4m3fn value, ties to even
    (the fp8 format of the [FA3-guide] fp8 listing): 3 mantissa bits,
    exponent bias 7, normal exponents -6..8, subnormal step 2^-9, largest
    finite value 448 (magnitudes beyond saturate to +-448, as a
    saturating conversion does). Used only by the report-only diagnostic
    below; the oracle proper never rounds to e4m3."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)                       # below 2^-6: subnormal step
    step = np.exp2(e - 3)
    r = np.round(a / step) * step               # np.round: half to even
    r = np.minimum(r, 448.0)
    return np.where(a > 0, np.copysign(r, x), x)


def attention_fp8_p_e4m3(qc, kc, vc, s_q, s_k, s_v, scale, causal=False,
                         rows=None):
    """REPORT-ONLY diagnostic, never a parity gate: ``attention_fp8`` with
    the probabilities rounded to e4m3 before the product with V, as the
    [FA3-guide] fp8 listing casts P to fp8 before its P.V GEMM.

    P is taken relative to the row's global maximum (exp(S - m) in [0, 1],
    the three-pass form of [Capstone §2.1]), rounded with ``round_e4m3``,
    and O = round(P) V / sum(round(P)): the rounded weights divided by
    their own sum. LSE is that of ``attention_fp8`` (unrounded). The
    kernel's own rounding is of P against a running reference, so this is
    one plausible size of the rounding effect, printed beside the gate.
    """
    q = np.asarray(qc, dtype=np.float64) * float(s_q)
    k = np.asarray(kc, dtype=np.float64) * float(s_k)
    v = np.asarray(vc, dtype=np.float64) * float(s_v)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    group = Hq // Hkv
    if rows is None:
        rows = np.arange(Nq, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, Hq, rows.shape[0], d), dtype=np.float64)
    _, lse = attention(q, k, v, scale, causal=causal, rows=rows)
    vis = _visible(rows, Nq, Nk) if causal else None
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            S = scale * (q[b, h, rows, :] @ k[b, hk].T)
            if vis is not None:
                S = np.where(vis, S, -np.inf)
            m = np.max(S, axis=1)
            live = m > -np.inf
            Pr = np.zeros_like(S)
            Pr[live] = round_e4m3(np.exp(S[live] - m[live, None]))
            z = np.sum(Pr, axis=1)
            out[b, h, live] = (Pr[live] @ v[b, hk]) / z[live, None]
    return out, lse


# --------------------------------------------------------------------------
# Merge of partial results over disjoint key sets
# --------------------------------------------------------------------------
def merge_partials(o_parts, lse_parts):
    """Merge normalised partial outputs computed over disjoint key subsets.

    o_parts: [S, ..., d]; lse_parts: [S, ...] (natural-log LSE of each part,
    -inf for an empty part). This is the two-block merge of
    [Capstone §2.2 step 4] and appendix A Q1, applied to S parts whose O is
    already divided by its own l: with L = log sum_s exp(lse_s), the merged
    output is sum_s exp(lse_s - L) * O_s and the merged LSE is L.
    An all-empty set of parts gives O = 0, LSE = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = np.max(lse_parts, axis=0)
    live = m > -np.inf
    m_safe = np.where(live, m, 0.0)
    w = np.exp(lse_parts - m_safe[None])                 # exp(-inf) = 0
    tot = np.sum(w, axis=0)
    L = np.where(live, m_safe + np.log(np.where(live, tot, 1.0)), -np.inf)
    coef = np.where(live[None], w / np.where(live, tot, 1.0)[None], 0.0)
    o = np.sum(coef[..., None] * o_parts, axis=0)
    return o, L


# --------------------------------------------------------------------------
# Paged KV cache decode
# --------------------------------------------------------------------------
def gather_paged_kv(pool, block_table_row, seq_len, page_size):
    """Rebuild one request's contiguous cache from its pages [FA3-paged §3.2].

    pool: [num_pages, page_size, Hkv, d]; block_table_row: physical page of
    each logical page. Returns [Hkv, seq_len, d]: logical page p holds
    tokens p*page_size .. p*page_size+page_size-1; tokens at or beyond
    seq_len are not part of the context.
    """
    pool = np.asarray(pool)
    n = -(-int(seq_len) // int(page_size))
    if n == 0:
        return np.zeros((pool.shape[2], 0, pool.shape[3]), dtype=np.float64)
    pages = [np.asarray(pool[int(block_table_row[p])], dtype=np.float64)
             for p in range(n)]
    kv = np.concatenate(pages, axis=0)[: int(seq_len)]    # [L, Hkv, d]
    return np.transpose(kv, (1, 0, 2))


def paged_decode(q, k_pool, v_pool, block_table, seq_lens, page_size, scale):
    """One query token per request against its paged KV cache.

    q: [B, Hq, d]; pools: [num_pages, page_size, Hkv, d]; block_table:
    [B, max_pages] physical page ids; seq_lens: [B]. The single query sees
    every cached token of its request (no mask inside the context).
    Returns (O [B, Hq, d], LSE [B, Hq]) in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    out = np.zeros((B, Hq, d), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        K = gather_paged_kv(k_pool, block_table[b], seq_lens[b], page_size)
        V = gather_paged_kv(v_pool, block_table[b], seq_lens[b], page_size)
        o, s = attention(q[b][None, :, None, :], K[None], V[None], scale)
        out[b] = o[0, :, 0, :]
        lse[b] = s[0, :, 0]
    return out, lse


def paged_decode_fp8(q, k_codes, v_codes, s_k, s_v, block_table, seq_lens,
                     page_size, scale):
    """Paged decode over a cache stored as e4m3 codes with per-pool scales
    ([FA3-guide] fp8 listing's per-tensor scaling, [FA3-paged §3.2] pages):
    the cached values are code * s, multiplied out exactly in fp64, then
    ``paged_decode`` of those values."""
    kx = np.asarray(k_codes, dtype=np.float64) * float(s_k)
    vx = np.asarray(v_codes, dtype=np.float64) * float(s_v)
    return paged_decode(q, kx, vx, block_table, seq_lens, page_size, scale)


def paged_prefill(q, k_pool, v_pool, block_table, seq_lens, page_size, scale,
                  causal=True):
    """Chunked prefill against a paged cache ([FA3-paged §3.2] pages): the
    Nq queries of request r are its last Nq positions, so with the cache
    gathered back to [Hkv, L, d] this is ``attention`` with Nk = L, whose
    bottom-right causal alignment lets query i see keys j <= i + L - Nq.
    q: [B, Hq, Nq, d]. Returns (O [B, Hq, Nq, d], LSE [B, Hq, Nq])."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, Nq, d = q.shape
    out = np.zeros((B, Hq, Nq, d), dtype=np.float64)
    lse = np.full((B, Hq, Nq), -np.inf, dtype=np.float64)
    for b in range(B):
        K = gather_paged_kv(k_pool, block_table[b], seq_lens[b], page_size)
        V = gather_paged_kv(v_pool, block_table[b], seq_lens[b], page_size)
        o, s = attention(q[b][None], K[None], V[None], scale, causal=causal)
        out[b] = o[0]
        lse[b] = s[0]
    return out, lse


# --------------------------------------------------------------------------
# Attention backward (the gradient of the definition)
# --------------------------------------------------------------------------
def attention_backward(q, k, v, do, scale, causal=False):
    """Gradients of O = softmax(scale * Q K^T) V, fp64.

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d]; do: dL/dO, [B, Hq, Nq, d].
    Returns (dQ [B, Hq, Nq, d], dK [B, Hkv, Nk, d], dV [B, Hkv, Nk, d]).

    Per (b, h), with P the row softmax of the (masked) scaled scores, taken
    from the same three-pass softmax as ``attention``:
      dV  = P^T dO                              (O is linear in V)
      dP  = dO V^T
      dS  = P * (dP - rowsum(P * dP))           (the softmax Jacobian:
                                                 dP_ij -> P_ij (dP_ij - sum_k P_ik dP_ik))
      dQ  = scale * dS K,    dK = scale * dS^T Q
    Masked scores have P = 0 and so no gradient; a row that sees no key has
    zero gradients. A KV head shared by a group of query heads collects the
    sum of their dK and dV (the chain rule through the shared tensor).
    The forward statistics the GPU path saves (LSE) and its row sums
    rowsum(dO * O) are the same quantities up to rounding; the oracle does
    not use them.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if do.shape != q.shape or v.shape != k.shape or Hq % Hkv != 0:
        raise ValueError("shape mismatch")
    group = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if Nq == 0 or Nk == 0:
        return dq, dk, dv
    vis = _visible(np.arange(Nq), Nq, Nk) if causal else None
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            S = scale * (q[b, h] @ k[b, hk].T)                  # [Nq, Nk]
            if vis is not None:
                S = np.where(vis, S, -np.inf)
            m = np.max(S, axis=1)
            live = m > -np.inf
            E = np.zeros_like(S)
            E[live] = np.exp(S[live] - m[live, None])
            l = np.sum(E, axis=1)
            P = np.zeros_like(S)
            P[live] = E[live] / l[live, None]
            dv[b, hk] += P.T @ do[b, h]
            dP = do[b, h] @ v[b, hk].T
            dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
            dq[b, h] = scale * (dS @ k[b, hk])
            dk[b, hk] += scale * (dS.T @ q[b, h])
    return dq, dk, dv
