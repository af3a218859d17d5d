#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass of the whole path over its synthetic workloads:
  1. bf16 causal GQA prefill, B=1, Hq=32, Hkv=8, N=16384, d=128 (fa_fwd)
  2. paged-KV decode, 64 requests, lengths U{512..8192}, page 16,
     Hq=32, Hkv=8, d=128 (fa_paged_decode: split kernel + merge kernel)
  3. fp8 e4m3 prefill, B=2, H=16, N=8192, d=128, non-causal (fa_fwd)
  4. the backward of workload 1 (fa_bwd: dQ, dK, dV from O, LSE and a
     seeded dO)
  5. workload 2 over a cache stored as e4m3 codes (fa_paged_decode_fp8kv)
  6. the non-causal bf16 prefill B=4, H=16, N=2048, d=128, fused (fa_fwd)
     and as the pages' three-kernel contrast (fa_naive_attention)
  7. chunked prefill against the paged cache (fa_paged_prefill): 16
     requests, 512 new tokens each, caches of U{4096..8192} tokens
Inputs are seeded N(0,1) draws (seed 42) already resident in HBM when the
timed region starts. Each launch is bracketed by HIP events on the stream
it runs on; the step time is the wall time of K steps of legs 1-3 between
two device synchronisations. Legs 5-7 are timed afterwards in a phase of
their own, K launches each, and leg 4 (the backward) last, in another.

Prints ONE JSON line. `value` is the bf16 causal prefill throughput in
TFLOPS (algorithmic FLOPs: 4*d per visible (query, key) pair per query
head; causal counts N(N+1)/2 pairs). The decode, fp8 and backward legs are
reported in their own objects (GB/s of algorithmic KV bytes, TFLOPS; the
backward counts 10*d FLOPs per visible pair: five products).

Each compute leg states its fraction of the datasheet peak (quoted at
2.4 GHz) and, after the timed region, the shader clock it holds under its
own load (bench_clock.hip's probe on a side stream while the leg runs back
to back) with the fraction of the peak scaled to that clock.

cpu_baseline: the fp64 oracle on this host, before the GPU is touched: a
pool of one worker per core (at most 16) with one BLAS thread each, over
256-row blocks of the causal prefill (about 12 s of work) and every request
of the paged decode; core count and CPU model are stated.

--sweep (not part of the default run) measures instead the sequence sweep
of the capstone page's roofline lab (h = 32, d = 128, non-causal, N = 1K to
32K): the fused forward against the three-kernel contrast that writes S
and P to HBM, beside the page's roofline model of the two (traffic 8Nd +
8N^2 bytes per head for the contrast as its §1.1 derives, 8Nd for the
fused pass; FLOPs 4N^2 d + 3N^2) at this GPU's peaks; then the causal GQA
prefill of the headline (Hq = 32, Hkv = 8, d = 128) over the same lengths,
and the paged decode (Hq = 32, Hkv = 8, d = 128, page 16) from one long
request to many short ones; one JSON line with a row per point.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("prefill attention TFLOPS (% MFMA peak) + paged-decode HBM GB/s "
          "(% peak)")
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

PREFILL = "bf16_causal_gqa_b1_hq32_hkv8_n16384_d128"
NONCAUSAL = "bf16_b4_h16_n2048_d128"
FP8 = "fp8_b2_h16_n8192_d128"
DECODE = "paged_decode_r64_hq32_hkv8_d128_p16"


def prefill_flops(c):
    """4*d FLOPs per visible (query, key) pair per query head."""
    Nq, Nk = c["Nq"], c["Nk"]
    if c["causal"]:
        off = Nk - Nq
        pairs = sum(max(0, min(Nk, i + off + 1)) for i in range(Nq))
    else:
        pairs = Nq * Nk
    return 4.0 * c["d"] * pairs * c["Hq"] * c["B"]


def decode_bytes(di, Hkv, d, kv_elem_bytes=2):
    """K and V of every cached token read once per KV head (the query heads
    of a group share them), plus q, o, LSE and the block-table entries."""
    import torch
    L = di.seq_lens.to(torch.int64)
    kv = int(L.sum()) * Hkv * d * 2 * kv_elem_bytes
    B, Hq, _ = di.q.shape
    pages = int(((L + di.page_size - 1) // di.page_size).sum())
    return kv + B * Hq * d * 2 * 2 + B * Hq * 4 + pages * 4


class ClockProbe:
    """The shader clock a kernel holds under its own load: bench_clock.so's
    probe (one wave reading the shader-clock counter against the constant
    100 MHz counter) runs on a side stream while the kernel is launched back
    to back on the main stream. On this chip it agrees with the rocprofv3
    GRBM_COUNT clock of the same kernel to within about 2 %. None when the
    probe library has not been built."""

    def __init__(self, stream):
        import ctypes
        import torch
        self.ok = False
        path = os.path.join(ROOT, "bench_clock.so")
        try:
            lib = ctypes.CDLL(path)
            lib.bench_clock_probe.argtypes = [ctypes.c_void_p,
                                              ctypes.c_ulonglong,
                                              ctypes.c_void_p]
            lib.bench_clock_probe.restype = ctypes.c_int
            lib.bench_clock_wall_rate_khz.restype = ctypes.c_int
            self.khz = lib.bench_clock_wall_rate_khz()
            self.lib = lib
            self.stream = stream
            self.side = torch.cuda.Stream()        # default priority
            self.out = torch.zeros(2, dtype=torch.int64, device="cuda:0")
            self.ok = self.khz > 0
        except OSError as e:
            print(f"bench: no clock probe ({e})", file=sys.stderr)

    def measure(self, fn, seconds=0.25):
        """Mean shader clock (MHz) over `seconds` of fn() run back to back,
        and the window's length in ms."""
        import torch
        if not self.ok:
            return None, 0.0
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        done = torch.cuda.Event()
        rc = self.lib.bench_clock_probe(self.out.data_ptr(),
                                        int(seconds * self.khz * 1e3),
                                        self.side.cuda_stream)
        if rc != 0:
            return None, 0.0
        done.record(self.side)
        while not done.query():
            for _ in range(4):
                fn()
            self.stream.synchronize()
        torch.cuda.synchronize()
        cyc, ticks = self.out.tolist()
        if ticks <= 0:
            return None, 0.0
        return cyc / ticks * self.khz / 1e3, ticks / self.khz


DATASHEET_MHZ = 2400.0


def _at_clock(achieved, peak, mhz, n):
    """The fraction of the datasheet peak, and of the peak scaled to the
    measured shader clock."""
    d = {"clock_mhz": mhz, "clock_window_ms": n,
         "clock_source": "shader-clock probe (bench_clock.hip) on a side "
                         "stream while the kernel ran back to back, after "
                         "the timed region"}
    if mhz:
        d["peak_at_clock"] = peak * mhz / DATASHEET_MHZ
        d["frac_at_clock"] = achieved / d["peak_at_clock"]
    return d


def _launch_stats(samples):
    """Mean, median, min and max of one leg's per-launch times in ms."""
    return {"launch_ms_mean": statistics.mean(samples),
            "launch_ms_median": statistics.median(samples),
            "launch_ms_min": min(samples), "launch_ms_max": max(samples)}


def _src_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "exact_attention_28_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_key, sources):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or
    None when none exists or the kernel source changed since."""
    p = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(p) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != _src_hash(sources):
        return None
    return rec.get("bytes_per_launch")


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# Arrays the CPU-baseline workers read: set before the pool forks, so every
# worker inherits them and a task is only a pair of indices.
_CPU = {}


def _cpu_worker_init():
    # one BLAS thread per worker (the environment was set before the pool
    # started; this covers libraries that ignore it)
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # noqa: BLE001
        pass


def _cpu_ping(x):
    return x


def _cpu_prefill_item(task):
    """The oracle on one block of query rows of one query head of the causal
    prefill (with the head's whole K/V, as the oracle takes them)."""
    import oracle
    h, j = task
    q, k, v, G, R, scale = (_CPU[x] for x in ("q", "k", "v", "G", "R", "scale"))
    rows = np.arange(j * R, (j + 1) * R)
    t0 = time.perf_counter()
    oracle.attention(q[h][None, None], k[h // G][None, None],
                     v[h // G][None, None], scale, causal=True, rows=rows)
    return time.perf_counter() - t0


def _cpu_decode_item(r):
    """The oracle's paged decode of request r."""
    import oracle
    d = _CPU["dec"]
    t0 = time.perf_counter()
    oracle.paged_decode(d["q"][r:r + 1], d["kp"], d["vp"], d["bt"][r:r + 1],
                        d["sl"][r:r + 1], d["page"], d["scale"])
    return time.perf_counter() - t0


def cpu_baseline(prefill_inp, decode_inp, target_s=12.0, rows=256):
    """The fp64 oracle timed on this host's cores, on the same seeded arrays
    the GPU legs use: a pool of one worker per core (at most 16: the host
    share of one GPU), one BLAS thread each. Called before the GPU is
    touched (the workers are forked from this process).

    * prefill: blocks of `rows` query rows of the causal GQA prefill, spread
      over heads and row positions (a block at every row offset, so the
      causal work mix is the workload's), as many as take about target_s;
      the rate counts the algorithmic FLOPs of the rows computed.
    * decode: every request of the paged-decode workload, one task each;
      the rate counts the algorithmic bytes (K/V once per KV head + q, o,
      LSE, table entries), as the GPU figure does.
    """
    import multiprocessing as mp

    import oracle  # noqa: F401  (imported before the fork: workers inherit it)
    import torch
    import workloads as W
    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(affinity, 16))
    c = W.PREFILL_CONFIGS[PREFILL]
    N, d, Hq = c["Nq"], c["d"], c["Hq"]
    _CPU.update(q=W.as_f64(prefill_inp.q)[0], k=W.as_f64(prefill_inp.k)[0],
                v=W.as_f64(prefill_inp.v)[0], G=c["Hq"] // c["Hkv"], R=rows,
                scale=prefill_inp.scale)
    di = decode_inp
    _CPU["dec"] = dict(q=W.as_f64(di.q),
                       kp=di.k_pool.to(torch.float32).numpy(),
                       vp=di.v_pool.to(torch.float32).numpy(),
                       bt=di.block_table.numpy(), sl=di.seq_lens.numpy(),
                       page=di.page_size, scale=di.scale)
    saved = {k: os.environ.get(k) for k in
             ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    pool = mp.get_context("fork").Pool(workers, initializer=_cpu_worker_init)
    for k, val in saved.items():
        if val is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = val
    out = {"unit": "TFLOPS", "kind": "oracle", "cores": workers,
           "affinity_cores": affinity, "cpu_model": _cpu_model(),
           "blas_threads_per_worker": 1}
    try:
        pool.map(_cpu_ping, range(workers))   # every worker up before timing
        nblk = N // rows
        order = [(i % Hq, (i * 7) % nblk) for i in range(Hq * nblk)]
        # rounds of one task per worker until target_s has passed (one
        # untimed round first: page faults on the inherited arrays)
        pool.map(_cpu_prefill_item, order[:workers], chunksize=1)
        n_items, flops = 0, 0.0
        t0 = time.perf_counter()
        while n_items < len(order) and time.perf_counter() - t0 < target_s:
            tasks = order[n_items:n_items + workers]
            pool.map(_cpu_prefill_item, tasks, chunksize=1)
            n_items += len(tasks)
            flops += sum(4.0 * d * float(np.sum(np.arange(j * rows, (j + 1) * rows) + 1))
                         for _, j in tasks)
        el = time.perf_counter() - t0
        out.update({"value": flops / el / 1e12, "seconds": el,
                    "sample": f"fp64 oracle on {n_items} blocks of {rows} "
                              f"query rows of the causal GQA prefill N={N} "
                              f"d={d} (every row offset; {flops / 1e9:.1f} "
                              f"GFLOP in {el:.1f} s), {workers} workers x 1 "
                              f"BLAS thread"})
        nreq = di.q.shape[0]
        nbytes = decode_bytes(di, di.k_pool.shape[2], di.k_pool.shape[3])
        t0 = time.perf_counter()
        pool.map(_cpu_decode_item, range(nreq), chunksize=1)
        el = time.perf_counter() - t0
        out["decode"] = {"value": nbytes / el / 1e9, "unit": "GB/s",
                         "seconds": el,
                         "sample": f"fp64 oracle paged decode of all {nreq} "
                                   f"requests ({nbytes / 1e6:.1f} MB "
                                   f"algorithmic), {workers} workers"}
    finally:
        pool.terminate()
        pool.join()
        _CPU.clear()
    return out


def sweep(steps, warmup):
    """The capstone roofline lab's sweep (h = 32, d = 128, N = 1K..32K,
    non-causal, one sequence) measured: fused forward and the three-kernel
    contrast, HIP events around each launch, median of `steps`; the lab's
    traffic model at MI355X peaks beside each row. Inputs: seeded N(0,1)
    draws rounded to bf16 (the workloads module, seed 42)."""
    import torch
    import workloads as W
    import exact_attention_28_amd as fa
    fa.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    H, d = 32, 128
    rows = []
    for n in (1024, 2048, 4096, 8192, 16384, 32768):
        inp = W.prefill_inputs(1, H, H, n, n, d, dtype="bf16", causal=False,
                               seed=42)
        q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
        del inp
        of = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        on = torch.empty_like(of)
        lf = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        ln = torch.empty_like(lf)
        # the contrast's softmax holds a row in one workgroup: rows of at
        # most 16384 scores (the entry point refuses longer ones)
        with_naive = n <= 16384
        ws = torch.empty(fa.fa_naive_workspace_size(1, H, n, n) if with_naive
                         else 256, dtype=torch.uint8, device=dev)
        args_ = (1, H, H, n, n, d, d ** -0.5, False)
        calls = {"fused": lambda: fa.fa_fwd(q, k, v, of, lf, *args_,
                                            fa.FA_DTYPE_BF16, None, stream)}
        if with_naive:
            calls["naive"] = lambda: fa.fa_naive_attention(
                q, k, v, on, ln, *args_, ws, ws.numel(), stream)
        ms = {}
        for name, call in calls.items():
            for _ in range(warmup):
                call()
            torch.cuda.synchronize()
            ev = []
            for _ in range(steps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                call()
                e1.record(stream)
                ev.append((e0, e1))
            torch.cuda.synchronize()
            ms[name] = statistics.median(a.elapsed_time(b) for a, b in ev)
        diff = (float((of.float() - on.float()).abs().max()) if with_naive
                else None)
        del ws
        flops = 4.0 * n * n * d * H           # the two products
        flops_sm = 3.0 * n * n * H            # the softmax (reported apart)
        # the page's ledger (§1.1): Q, K, V, O once (8Nd bytes) and S, P
        # written and read once each at 2 bytes an element (8N^2 bytes)
        b_naive = H * (8 * n * d + 8 * n * n)
        b_fused = H * (8 * n * d)
        t_c = (flops + flops_sm) / (PEAK_BF16_TFLOPS * 1e12)
        model = max(t_c, b_naive / (PEAK_HBM_GBS * 1e9)) / max(
            t_c, b_fused / (PEAK_HBM_GBS * 1e9))
        # the same model as the page's lab script evaluates it: its A100
        # figures (312 TFLOPS, 2039 GB/s) and its byte count, which doubles
        # the §1.1 ledger
        t_ca = (flops + flops_sm) / 312e12
        model_lab = max(t_ca, 2 * b_naive / 2039e9) / max(t_ca,
                                                          b_fused / 2039e9)
        tn = ms.get("naive")
        rows.append({
            "N": n, "fused_ms": ms["fused"], "naive_ms": tn,
            "fused_tflops": flops / (ms["fused"] * 1e-3) / 1e12,
            "fused_frac_bf16_peak": flops / (ms["fused"] * 1e-3) / 1e12 /
            PEAK_BF16_TFLOPS,
            "naive_tflops": flops / (tn * 1e-3) / 1e12 if tn else None,
            "naive_ledger_bytes": b_naive,
            "naive_ledger_GB/s": b_naive / (tn * 1e-3) / 1e9 if tn else None,
            "fused_ledger_bytes": b_fused,
            "speedup_measured": tn / ms["fused"] if tn else None,
            "speedup_model_mi355x": model,
            "speedup_model_lab_a100": model_lab,
            "max_abs_fused_minus_naive": diff,
        })
        print(f"bench sweep: N={n} fused {ms['fused']:.3f} ms"
              + (f", naive {tn:.3f} ms ({tn / ms['fused']:.2f}x, model "
                 f"{model:.2f}x), |fused - naive| <= {diff:.2e}" if tn else
                 f" (model speedup {model:.2f}x; no contrast past 16384)"),
              file=sys.stderr, flush=True)
        del q, k, v, of, on, lf, ln
        torch.cuda.empty_cache()

    def median_ms(call):
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        ev = []
        for _ in range(steps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) for a, b in ev)

    # the headline's causal GQA prefill over sequence length
    causal_rows = []
    for n in (1024, 2048, 4096, 8192, 16384, 32768):
        inp = W.prefill_inputs(1, 32, 8, n, n, d, dtype="bf16", causal=True,
                               seed=42)
        q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
        del inp
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        t = median_ms(lambda: fa.fa_fwd(q, k, v, o, lse, 1, 32, 8, n, n, d,
                                         d ** -0.5, True, fa.FA_DTYPE_BF16,
                                         None, stream))
        flops = 4.0 * d * 32 * n * (n + 1) / 2
        causal_rows.append({"N": n, "ms": t,
                            "tflops": flops / (t * 1e-3) / 1e12,
                            "frac_bf16_peak": flops / (t * 1e-3) / 1e12 /
                            PEAK_BF16_TFLOPS})
        print(f"bench sweep: causal GQA N={n} {t:.3f} ms "
              f"{flops / (t * 1e-3) / 1e12:.0f} TFLOP/s", file=sys.stderr,
              flush=True)
        del q, k, v, o, lse
        torch.cuda.empty_cache()

    # the paged decode: one long request to many short ones
    decode_rows = []
    for nreq, length in ((1, 32768), (1, 131072), (8, 16384), (64, 4096),
                         (256, 1024), (512, 512)):
        di = W.decode_inputs(nreq, 32, 8, d, lens=[length] * nreq, seed=42)
        q = di.q.to(dev)
        kp, vp = di.k_pool.to(dev), di.v_pool.to(dev)
        bt, sl = di.block_table.to(dev), di.seq_lens.to(dev)
        npages, page, hkv, _ = kp.shape
        maxp = bt.shape[1]
        ws = torch.empty(fa.fa_paged_decode_workspace_size(
            nreq, 32, hkv, d, maxp, page, 0), dtype=torch.uint8, device=dev)
        od = torch.empty((nreq, 32, d), dtype=torch.bfloat16, device=dev)
        ld = torch.empty((nreq, 32), dtype=torch.float32, device=dev)
        t = median_ms(lambda: fa.fa_paged_decode(
            q, kp, vp, bt, sl, page, npages, nreq, 32, hkv, d, maxp, di.scale,
            od, ld, ws, ws.numel(), 0, stream))
        nbytes = decode_bytes(di, hkv, d)
        decode_rows.append({"requests": nreq, "tokens_each": length,
                            "ms": t, "bytes": nbytes,
                            "GB/s": nbytes / (t * 1e-3) / 1e9,
                            "frac_hbm_peak": nbytes / (t * 1e-3) / 1e9 /
                            PEAK_HBM_GBS})
        print(f"bench sweep: decode {nreq} x {length} {t:.4f} ms "
              f"{nbytes / (t * 1e-3) / 1e9:.0f} GB/s", file=sys.stderr,
              flush=True)
        del di, q, kp, vp, bt, sl, ws, od, ld
        torch.cuda.empty_cache()
    print(json.dumps({
        "metric": "fused vs three-kernel attention forward over sequence "
                  "length (capstone roofline lab sweep)",
        "unit": "ms", "higher_is_better": False, "n_gpus": 1,
        "steps": steps, "warmup": warmup, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "B=1 H=32 d=128 non-causal N=1K..32K; causal "
                               "GQA Hq=32 Hkv=8 d=128 N=1K..32K; paged "
                               "decode Hq=32 Hkv=8 d=128 page 16, 1x32K .. "
                               "512x512 tokens",
                   "seed": 42},
        "sweep": rows, "causal_gqa": causal_rows, "decode": decode_rows}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--clock-seconds", type=float, default=0.25,
                    help="seconds of back-to-back launches per leg for the "
                    "shader-clock probe after the timed region (0: skip, "
                    "for profiling runs)")
    ap.add_argument("--legs",
                    default="prefill,decode,fp8,bwd,decode8,noncausal,naive,"
                    "chunked",
                    help="comma list of legs to run (profiling runs)")
    ap.add_argument("--sweep", action="store_true",
                    help="only the sequence sweep of the capstone roofline "
                    "lab: fused vs three-kernel forward, N = 1K..32K")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus "
              f"{args.gpus}); multi-GPU sharding is not implemented",
              file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        sweep(args.steps, args.warmup)
        return

    import torch
    import workloads as W
    legs = [x for x in args.legs.split(",") if x]

    # host inputs first; the CPU oracle baseline runs on them before the GPU
    # is touched (its worker pool is forked from this process)
    host = {}
    if "prefill" in legs or "bwd" in legs:
        host["prefill"] = W.prefill_config(PREFILL)
    if "decode" in legs:
        host["decode"] = W.decode_config(DECODE)
    cpu = None
    if not args.no_cpu_baseline and "prefill" in legs and "decode" in legs:
        print("bench: timing the CPU oracle baseline", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(host["prefill"], host["decode"])
        print(f"bench: CPU oracle {cpu['value'] * 1e3:.1f} GFLOP/s, decode "
              f"{cpu['decode']['value']:.2f} GB/s", file=sys.stderr,
              flush=True)

    import exact_attention_28_amd as fa
    fa.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    calls = {}
    info = {}
    if "prefill" in legs:
        c = W.PREFILL_CONFIGS[PREFILL]
        inp = host["prefill"]
        q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        calls["prefill"] = lambda q=q, k=k, v=v, o=o, lse=lse, c=c, inp=inp: fa.fa_fwd(
            q, k, v, o, lse, c["B"], c["Hq"], c["Hkv"], c["Nq"], c["Nk"],
            c["d"], inp.scale, True, fa.FA_DTYPE_BF16, None, stream)
        info["prefill"] = dict(flops=prefill_flops(c), cfg=c)
    if "decode" in legs:
        c = W.DECODE_CONFIGS[DECODE]
        di = host["decode"]
        q = di.q.to(dev)
        kp, vp = di.k_pool.to(dev), di.v_pool.to(dev)
        bt, sl = di.block_table.to(dev), di.seq_lens.to(dev)
        B, Hq, d = q.shape
        npages, page, Hkv, _ = kp.shape
        maxp = bt.shape[1]
        need = fa.fa_paged_decode_workspace_size(B, Hq, Hkv, d, maxp, page, 0)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        od = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev)
        ld = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        calls["decode"] = lambda: fa.fa_paged_decode(
            q, kp, vp, bt, sl, page, npages, B, Hq, Hkv, d, maxp, di.scale,
            od, ld, ws, ws.numel(), 0, stream)
        info["decode"] = dict(bytes=decode_bytes(di, Hkv, d), cfg=c,
                              kv_tokens=int(di.seq_lens.sum()))
    if "copy" in legs:
        # plain copy of a known size: reference reading for the HBM counters
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        calls["copy"] = lambda: torch.mul(src, 1.0, out=dst)
        info["copy"] = dict(bytes=2 * nbytes)
    if "fp8" in legs:
        c = W.PREFILL_CONFIGS[FP8]
        inp = W.prefill_config(FP8)
        q8, k8, v8 = (t.to(dev) for t in (inp.q, inp.k, inp.v))
        o8 = torch.empty(q8.shape, dtype=torch.bfloat16, device=dev)
        l8 = torch.empty(q8.shape[:3], dtype=torch.float32, device=dev)
        calls["fp8"] = lambda c=c, inp=inp: fa.fa_fwd(
            q8, k8, v8, o8, l8, c["B"], c["Hq"], c["Hkv"], c["Nq"], c["Nk"],
            c["d"], inp.scale, False, fa.FA_DTYPE_FP8_E4M3, inp.descale,
            stream)
        info["fp8"] = dict(flops=prefill_flops(c), cfg=c)
    if "bwd" in legs:
        # backward of the causal GQA prefill: O and LSE from one forward
        # call outside the timed region, dO seeded
        cb = W.PREFILL_CONFIGS[PREFILL]
        ib = host["prefill"]
        qb, kb, vb = (t.to(dev) for t in (ib.q, ib.k, ib.v))
        gb = W.upstream_grad(tuple(ib.q.shape), seed=43).to(dev)
        ob = torch.empty(qb.shape, dtype=torch.bfloat16, device=dev)
        lb = torch.empty(qb.shape[:3], dtype=torch.float32, device=dev)
        fa.fa_fwd(qb, kb, vb, ob, lb, cb["B"], cb["Hq"], cb["Hkv"], cb["Nq"],
                  cb["Nk"], cb["d"], ib.scale, True, fa.FA_DTYPE_BF16, None,
                  stream)
        dqb, dkb, dvb = (torch.empty_like(t) for t in (qb, kb, vb))
        wsb = torch.empty(fa.fa_bwd_workspace_size(cb["B"], cb["Hq"], cb["Nq"]),
                          dtype=torch.uint8, device=dev)
        calls["bwd"] = lambda cb=cb, ib=ib: fa.fa_bwd(
            qb, kb, vb, ob, gb, lb, dqb, dkb, dvb, cb["B"], cb["Hq"],
            cb["Hkv"], cb["Nq"], cb["Nk"], cb["d"], ib.scale, True,
            fa.FA_DTYPE_BF16, wsb, wsb.numel(), stream)
        # five products of 2*d FLOPs per visible pair (S re-computed, dP,
        # dV, dQ, dK): 2.5 times the forward's work
        info["bwd"] = dict(flops=2.5 * prefill_flops(cb), cfg=cb)
    if "decode8" in legs:
        # the same decode over the cache stored as e4m3 codes + two scales
        d8 = W.decode_config(DECODE, kv_dtype="fp8")
        q8d = d8.q.to(dev)
        kp8, vp8 = d8.k_pool.to(dev), d8.v_pool.to(dev)
        bt8, sl8 = d8.block_table.to(dev), d8.seq_lens.to(dev)
        B8, Hq8, dd8 = q8d.shape
        np8, pg8, Hkv8, _ = kp8.shape
        mp8 = bt8.shape[1]
        ws8 = torch.empty(fa.fa_paged_decode_workspace_size(
            B8, Hq8, Hkv8, dd8, mp8, pg8, 0), dtype=torch.uint8, device=dev)
        od8 = torch.empty((B8, Hq8, dd8), dtype=torch.bfloat16, device=dev)
        ld8 = torch.empty((B8, Hq8), dtype=torch.float32, device=dev)
        calls["decode8"] = lambda: fa.fa_paged_decode_fp8kv(
            q8d, kp8, vp8, bt8, sl8, pg8, np8, B8, Hq8, Hkv8, dd8, mp8,
            d8.scale, d8.kv_descale, od8, ld8, ws8, ws8.numel(), 0, stream)
        info["decode8"] = dict(bytes=decode_bytes(d8, Hkv8, dd8, 1),
                               kv_tokens=int(d8.seq_lens.sum()))
    if "noncausal" in legs or "naive" in legs:
        # the non-causal bf16 prefill, fused and as the pages' three-kernel
        # contrast (S and P through HBM)
        cn = W.PREFILL_CONFIGS[NONCAUSAL]
        i_n = W.prefill_config(NONCAUSAL)
        qn, kn, vn = (t.to(dev) for t in (i_n.q, i_n.k, i_n.v))
        on = torch.empty(qn.shape, dtype=torch.bfloat16, device=dev)
        ln = torch.empty(qn.shape[:3], dtype=torch.float32, device=dev)
        args_n = (cn["B"], cn["Hq"], cn["Hkv"], cn["Nq"], cn["Nk"], cn["d"],
                  i_n.scale, False)
        if "noncausal" in legs:
            calls["noncausal"] = lambda: fa.fa_fwd(
                qn, kn, vn, on, ln, *args_n, fa.FA_DTYPE_BF16, None, stream)
            info["noncausal"] = dict(flops=prefill_flops(cn), cfg=cn)
        if "naive" in legs:
            wsn = torch.empty(fa.fa_naive_workspace_size(
                cn["B"], cn["Hq"], cn["Nq"], cn["Nk"]), dtype=torch.uint8,
                device=dev)
            calls["naive"] = lambda: fa.fa_naive_attention(
                qn, kn, vn, on, ln, *args_n, wsn, wsn.numel(), stream)
            info["naive"] = dict(flops=prefill_flops(cn), cfg=cn)
    if "chunked" in legs:
        # chunked prefill: a 512-token chunk for each of 16 requests against
        # paged caches of U{4096..8192} tokens (the chunk's own positions
        # included), Hq=32, Hkv=8, d=128, causal
        import numpy as np
        lens_c = np.random.default_rng(42).integers(4096, 8192, size=16,
                                                    endpoint=True)
        dc = W.paged_prefill_inputs(16, 32, 8, 128, 512, lens=list(lens_c),
                                    max_pages=512, seed=42)
        qc = dc.q.to(dev)
        kpc, vpc = dc.k_pool.to(dev), dc.v_pool.to(dev)
        btc, slc = dc.block_table.to(dev), dc.seq_lens.to(dev)
        oc = torch.empty(qc.shape, dtype=torch.bfloat16, device=dev)
        lc = torch.empty(qc.shape[:3], dtype=torch.float32, device=dev)
        calls["chunked"] = lambda: fa.fa_paged_prefill(
            qc, kpc, vpc, btc, slc, 16, kpc.shape[0], 16, 32, 8, 512, 128,
            btc.shape[1], dc.scale, True, oc, lc, stream)
        pairs = sum(sum(min(int(L), i + int(L) - 512 + 1) for i in range(512))
                    for L in lens_c)
        info["chunked"] = dict(flops=4.0 * 128 * pairs * 32)
    torch.cuda.synchronize()
    print(f"bench: inputs resident, legs={legs}", file=sys.stderr, flush=True)

    # the step: the forward hot path (prefill, decode, fp8). The other
    # forward legs are timed after it in a phase of their own, and the
    # backward last, in another: its heat and power draw (and the caches it
    # leaves behind) do not change what the forward legs run at
    order = [x for x in ("prefill", "decode", "fp8", "copy") if x in calls]
    phases = [[x for x in ("decode8", "noncausal", "naive", "chunked")
               if x in calls], [x for x in ("bwd",) if x in calls]]

    def timed(names, steps):
        ev = {n: [] for n in names}
        for _ in range(steps):
            for name in names:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                calls[name]()
                e1.record(stream)
                ev[name].append((e0, e1))
        return ev

    for _ in range(args.warmup):
        for name in order:
            calls[name]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev = timed(order, args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for extra in phases:
        if not extra:
            continue
        for _ in range(args.warmup):
            for name in extra:
                calls[name]()
        torch.cuda.synchronize()
        ev.update(timed(extra, args.steps))
        torch.cuda.synchronize()
        order = order + extra
    ms = {n: [a.elapsed_time(b) for a, b in ev[n]] for n in order}
    # the shader clock each kernel holds under its own load, sampled while
    # it runs back to back (outside the timed region)
    clock = {n: (None, 0.0) for n in order}
    if args.clock_seconds > 0:
        probe = ClockProbe(stream)
        for name in order:
            if name != "naive":
                clock[name] = probe.measure(calls[name], args.clock_seconds)
    print("bench: clocks " + ", ".join(
        f"{n}={c[0]:.0f}MHz" for n, c in clock.items() if c[0]),
        file=sys.stderr, flush=True)
    print("bench: timed region done " + ", ".join(
        f"{n}={statistics.mean(ms[n]):.3f}ms" for n in order),
        file=sys.stderr, flush=True)

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic (seeded N(0,1), no dataset)"}
    workload = []
    if "prefill" in order:
        c = info["prefill"]["cfg"]
        t = statistics.mean(ms["prefill"]) / 1e3
        tf = info["prefill"]["flops"] / t / 1e12
        out["value"] = tf
        out["unit"] = "TFLOPS"
        out["roofline"] = {
            "kernel": "fwd_bf16_pp_kernel<causal>",
            "bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
            "traffic": _traffic("fwd_bf16_causal_n16384",
                                ["fa_fwd_bf16_pp.hip", "fa_pp_asm.h",
                                 "fa_device.h"]),
            "algorithmic_gflop_per_launch": info["prefill"]["flops"] / 1e9,
            # the pages' 3 softmax FLOPs per score, kept out of TFLOPS
            "softmax_gflop_per_launch": 0.75 * info["prefill"]["flops"]
            / c["d"] / 1e9,
            **_at_clock(tf, PEAK_BF16_TFLOPS, *clock["prefill"]),
            **_launch_stats(ms["prefill"])}
        workload.append(f"bf16 causal GQA prefill B={c['B']} Hq={c['Hq']} "
                        f"Hkv={c['Hkv']} N={c['Nq']} d={c['d']}")
    if "decode" in order:
        c = info["decode"]["cfg"]
        t = statistics.mean(ms["decode"]) / 1e3
        gbs = info["decode"]["bytes"] / t / 1e9
        out["decode"] = {
            "value": gbs, "unit": "GB/s", "frac_hbm_peak": gbs / PEAK_HBM_GBS,
            "roofline": {"kernel": "decode_kernel + decode_merge_kernel",
                         "bound": "hbm", "achieved": gbs,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS,
                         "traffic": _traffic("decode_r64",
                                             ["fa_decode.hip", "fa_device.h"]),
                         # HBM bandwidth does not scale with the shader
                         # clock; the clock is reported for reference
                         "clock_mhz": clock["decode"][0]},
            "algorithmic_bytes": info["decode"]["bytes"],
            "kv_tokens": info["decode"]["kv_tokens"],
            **_launch_stats(ms["decode"])}
        workload.append(f"paged decode {c['n_req']} requests L~U{{{c['len_min']}.."
                        f"{c['len_max']}}} page {c['page_size']} Hq={c['Hq']} "
                        f"Hkv={c['Hkv']} d={c['d']}")
        if "value" not in out:
            out["value"], out["unit"] = gbs, "GB/s"
    if "fp8" in order:
        c = info["fp8"]["cfg"]
        t = statistics.mean(ms["fp8"]) / 1e3
        tf = info["fp8"]["flops"] / t / 1e12
        out["fp8_prefill"] = {
            "value": tf, "unit": "TFLOPS", "frac_fp8_peak": tf / PEAK_FP8_TFLOPS,
            **_at_clock(tf, PEAK_FP8_TFLOPS, *clock["fp8"]),
            **_launch_stats(ms["fp8"])}
        workload.append(f"fp8 e4m3 prefill B={c['B']} H={c['Hq']} N={c['Nq']} "
                        f"d={c['d']}")
        if "value" not in out:
            out["value"], out["unit"] = tf, "TFLOPS"
    if "bwd" in order:
        c = info["bwd"]["cfg"]
        t = statistics.mean(ms["bwd"]) / 1e3
        tf = info["bwd"]["flops"] / t / 1e12
        out["backward"] = {
            "value": tf, "unit": "TFLOPS", "frac_bf16_peak": tf / PEAK_BF16_TFLOPS,
            "algorithmic_gflop_per_launch": info["bwd"]["flops"] / 1e9,
            "kernels": "bwd_prep_kernel + bwd_dkdv_kernel + bwd_dq_kernel",
            **_at_clock(tf, PEAK_BF16_TFLOPS, *clock["bwd"]),
            **_launch_stats(ms["bwd"])}
        workload.append(f"bf16 causal GQA backward B={c['B']} Hq={c['Hq']} "
                        f"Hkv={c['Hkv']} N={c['Nq']} d={c['d']}")
        if "value" not in out:
            out["value"], out["unit"] = tf, "TFLOPS"
    if "decode8" in order:
        t = statistics.mean(ms["decode8"]) / 1e3
        gbs = info["decode8"]["bytes"] / t / 1e9
        out["decode_fp8_cache"] = {
            "value": gbs, "unit": "GB/s", "frac_hbm_peak": gbs / PEAK_HBM_GBS,
            "kernel": "decode_kernel<e4m3 cache> + decode_merge_kernel",
            "algorithmic_bytes": info["decode8"]["bytes"],
            "tokens_per_s": info["decode8"]["kv_tokens"] / t,
            "clock_mhz": clock["decode8"][0],
            **_launch_stats(ms["decode8"])}
        workload.append("paged decode over an e4m3 cache (same requests)")
        if "value" not in out:
            out["value"], out["unit"] = gbs, "GB/s"
    for leg in ("noncausal", "naive"):
        if leg not in order:
            continue
        c = info[leg]["cfg"]
        t = statistics.mean(ms[leg]) / 1e3
        tf = info[leg]["flops"] / t / 1e12
        heads = c["B"] * c["Hq"]
        N, d = c["Nq"], c["d"]
        entry = {"value": tf, "unit": "TFLOPS", **_launch_stats(ms[leg])}
        if leg in clock:
            entry["clock_mhz"] = clock[leg][0]
        if leg == "naive":
            # the pages' traffic ledger, 8Nd + 8N^2 bytes per head
            entry["ledger_bytes"] = heads * (8 * N * d + 8 * N * N)
            entry["ledger_GB/s"] = entry["ledger_bytes"] / t / 1e9
            entry["kernels"] = ("naive_scores_kernel + "
                                "naive_softmax_wave_kernel + naive_pv_kernel")
        else:
            entry["ledger_bytes"] = heads * 8 * N * d
        out["bf16_noncausal_" + leg if leg == "naive" else
            "bf16_noncausal_fused"] = entry
        workload.append(f"bf16 prefill B={c['B']} H={c['Hq']} N={N} d={d} "
                        f"({'three-kernel contrast' if leg == 'naive' else 'fused'})")
    if "chunked" in order:
        t = statistics.mean(ms["chunked"]) / 1e3
        tf = info["chunked"]["flops"] / t / 1e12
        out["chunked_prefill"] = {
            "value": tf, "unit": "TFLOPS", "frac_bf16_peak": tf / PEAK_BF16_TFLOPS,
            "kernel": "fwd_bf16_pp_kernel<causal, paged>",
            **_at_clock(tf, PEAK_BF16_TFLOPS, *clock["chunked"]),
            **_launch_stats(ms["chunked"])}
        workload.append("chunked prefill 16 requests x 512 new tokens, paged "
                        "cache U{4096..8192}, Hq=32 Hkv=8 d=128")
        if "value" not in out:
            out["value"], out["unit"] = tf, "TFLOPS"
    if "copy" in order:
        t = statistics.mean(ms["copy"]) / 1e3
        out["copy_calibration"] = {"bytes_per_launch": info["copy"]["bytes"],
                                   "GB/s": info["copy"]["bytes"] / t / 1e9,
                                   **_launch_stats(ms["copy"])}
        if "value" not in out:
            out["value"], out["unit"] = info["copy"]["bytes"] / t / 1e9, "GB/s"
    out["config"] = {"workload": " + ".join(workload), "seed": 42,
                     "parallelism": "single GPU"}
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
