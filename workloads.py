"""Seeded synthetic inputs shared by the tests, the bench and smoke().

This module holds no attention arithmetic. It only draws random numbers and
rounds them to the storage formats the kernels read (bf16, OCP float8
e4m3fn with a per-tensor fp32 scale), using torch's own casts. Both the
fp64 oracle and the HIP library consume what it returns; neither is
imported here.

Shapes and distributions follow the workloads the attention pages study
(prefill at head dimension 64/128, long causal context, a paged decode
batch): i.i.d. N(0, 1) entries, seed 42 by default (the seed of the tiled
FA2 lab of the capstone page, lab 3).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

E4M3_MAX = 448.0          # largest finite OCP e4m3fn value

# The five workloads. Sizes are the real ones; tests also use reduced
# copies of the same recipes.
PREFILL_CONFIGS = {
    # single head, fp32, Nq = Nk = 256, d = 64
    "f32_n256_d64": dict(B=1, Hq=1, Hkv=1, Nq=256, Nk=256, d=64,
                         causal=False, dtype="f32"),
    # bf16 non-causal prefill
    "bf16_b4_h16_n2048_d128": dict(B=4, Hq=16, Hkv=16, Nq=2048, Nk=2048,
                                   d=128, causal=False, dtype="bf16"),
    # bf16 causal long context with grouped-query attention
    "bf16_causal_gqa_b1_hq32_hkv8_n16384_d128": dict(
        B=1, Hq=32, Hkv=8, Nq=16384, Nk=16384, d=128, causal=True,
        dtype="bf16"),
    # fp8 e4m3 prefill
    "fp8_b2_h16_n8192_d128": dict(B=2, Hq=16, Hkv=16, Nq=8192, Nk=8192,
                                  d=128, causal=False, dtype="fp8"),
}
DECODE_CONFIGS = {
    "paged_decode_r64_hq32_hkv8_d128_p16": dict(
        n_req=64, Hq=32, Hkv=8, d=128, page_size=16, len_min=512,
        len_max=8192),
}


def _to_storage(x: np.ndarray, dtype: str):
    """fp32 numpy -> torch CPU tensor in the storage dtype (+ scale)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "f32":
        return t, None
    if dtype == "bf16":
        return t.to(torch.bfloat16), None         # round to nearest even
    if dtype == "fp8":
        amax = float(t.abs().max()) if t.numel() else 0.0
        s = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
        y = torch.clamp(t / torch.tensor(s, dtype=torch.float32),
                        -E4M3_MAX, E4M3_MAX)
        return y.to(torch.float8_e4m3fn), float(s)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass
class PrefillInputs:
    q: torch.Tensor            # [B, Hq, Nq, d] storage dtype (CPU)
    k: torch.Tensor            # [B, Hkv, Nk, d]
    v: torch.Tensor
    scale: float               # softmax scale, 1/sqrt(d)
    causal: bool
    dtype: str                 # "f32" | "bf16" | "fp8"
    descale: tuple | None      # (s_q, s_k, s_v) for fp8, else None


def prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dtype="bf16", causal=False,
                   seed=42, scale=None) -> PrefillInputs:
    """Q, K, V i.i.d. N(0,1) in fp32 drawn in the order Q, K, V, then cast."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Nq, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    tq, sq = _to_storage(q, dtype)
    tk, sk = _to_storage(k, dtype)
    tv, sv = _to_storage(v, dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    descale = (sq, sk, sv) if dtype == "fp8" else None
    return PrefillInputs(tq, tk, tv, float(scale), bool(causal), dtype,
                         descale)


def prefill_config(name, seed=42) -> PrefillInputs:
    c = PREFILL_CONFIGS[name]
    return prefill_inputs(c["B"], c["Hq"], c["Hkv"], c["Nq"], c["Nk"],
                          c["d"], dtype=c["dtype"], causal=c["causal"],
                          seed=seed)


@dataclass
class DecodeInputs:
    q: torch.Tensor            # [B, Hq, d] bf16
    k_pool: torch.Tensor       # [num_pages, page_size, Hkv, d] bf16
    v_pool: torch.Tensor
    block_table: torch.Tensor  # [B, max_pages] int32, unused entries -1
    seq_lens: torch.Tensor     # [B] int32
    page_size: int
    scale: float
    kv_descale: tuple | None = None   # (s_k, s_v) for an e4m3 cache


POISON = 1.0e4   # finite filler for token slots past a request's length


def decode_inputs(n_req, Hq, Hkv, d, page_size=16, len_min=512,
                  len_max=8192, seed=42, max_pages=None, lens=None,
                  extra_pages=0, kv_dtype="bf16") -> DecodeInputs:
    """A paged KV cache for n_req requests, one query token each.

    Draw order: lengths ~ U{len_min..len_max} (unless ``lens`` is given),
    q ~ N(0,1), K pool, V pool ~ N(0,1), the page permutation, the poison
    signs. Logical page p of request r (request-major order) lives in the
    physical slot given by a seeded permutation of all pages. Slots of the
    last page beyond the request's length hold +/-1e4 so any masking error
    is gross. ``extra_pages`` adds never-referenced pages (also poisoned).

    kv_dtype "fp8": the pools are stored as e4m3 codes with one fp32 scale
    per pool (amax / 448 of the drawn values), and the poison is the
    largest finite code (+/-448): finite, so 0 * poison stays 0.
    """
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(len_min, len_max, size=n_req, endpoint=True)
    lens = np.asarray(lens, dtype=np.int64)
    n_pages = -(-lens // page_size)
    total = int(n_pages.sum()) + int(extra_pages)
    if max_pages is None:
        max_pages = max(1, -(-max(int(len_max), int(lens.max(initial=0)))
                            // page_size))
    q = rng.standard_normal((n_req, Hq, d), dtype=np.float32)
    kp = rng.standard_normal((total, page_size, Hkv, d), dtype=np.float32)
    vp = rng.standard_normal((total, page_size, Hkv, d), dtype=np.float32)
    perm = rng.permutation(total)
    poison = POISON
    kv_descale = None
    if kv_dtype == "fp8":
        scales = []
        for pool in (kp, vp):
            amax = float(np.max(np.abs(pool))) if pool.size else 0.0
            sc = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
            pool /= sc                      # now in code units
            scales.append(float(sc))
        kv_descale = tuple(scales)
        poison = E4M3_MAX
    elif kv_dtype != "bf16":
        raise ValueError(f"unknown kv_dtype {kv_dtype!r}")
    table = np.full((n_req, max_pages), -1, dtype=np.int32)
    slot = 0
    for r in range(n_req):
        for p in range(int(n_pages[r])):
            table[r, p] = perm[slot]
            slot += 1
        tail = int(lens[r]) - (int(n_pages[r]) - 1) * page_size
        if n_pages[r] > 0 and tail < page_size:
            phys = table[r, n_pages[r] - 1]
            sign = rng.choice(np.array([-1.0, 1.0], dtype=np.float32),
                              size=(page_size - tail, Hkv, d))
            kp[phys, tail:] = poison * sign
            vp[phys, tail:] = -poison * sign
    for p in perm[slot:]:                      # unreferenced pages
        kp[p] = poison
        vp[p] = -poison
    if kv_dtype == "fp8":
        def store(x):
            t = torch.from_numpy(x)
            return torch.clamp(t, -E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    else:
        def store(x):
            return torch.from_numpy(x).to(torch.bfloat16)
    return DecodeInputs(
        q=torch.from_numpy(q).to(torch.bfloat16),
        k_pool=store(kp),
        v_pool=store(vp),
        block_table=torch.from_numpy(table),
        seq_lens=torch.from_numpy(lens.astype(np.int32)),
        page_size=int(page_size),
        scale=1.0 / math.sqrt(d),
        kv_descale=kv_descale,
    )


def decode_config(name, seed=42, kv_dtype="bf16") -> DecodeInputs:
    c = DECODE_CONFIGS[name]
    return decode_inputs(c["n_req"], c["Hq"], c["Hkv"], c["d"],
                         page_size=c["page_size"], len_min=c["len_min"],
                         len_max=c["len_max"], seed=seed, kv_dtype=kv_dtype)


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a storage tensor to fp64 numpy (values unchanged)."""
    return t.to(torch.float64).numpy()


def upstream_grad(shape, seed=4242, dtype="bf16") -> torch.Tensor:
    """dL/dO for the backward tests: i.i.d. N(0, 1) in fp32, cast."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(tuple(shape), dtype=np.float32)
    t, _ = _to_storage(g, dtype)
    return t


def paged_prefill_inputs(n_req, Hq, Hkv, d, Nq, lens, max_pages=None,
                         seed=42, extra_pages=0):
    """A paged cache (the decode recipe: K/V pools N(0,1) in bf16, seeded
    page permutation, poisoned tail slots) plus Nq new query tokens per
    request, q [n_req, Hq, Nq, d] ~ N(0,1) bf16 drawn from seed + 1."""
    di = decode_inputs(n_req, Hq, Hkv, d, lens=lens, max_pages=max_pages,
                       seed=seed, extra_pages=extra_pages)
    rng = np.random.default_rng(seed + 1)
    q = rng.standard_normal((n_req, Hq, Nq, d), dtype=np.float32)
    di.q = torch.from_numpy(q).to(torch.bfloat16)
    return di
