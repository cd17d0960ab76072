#!/usr/bin/env python3
"""Benchmark of BAM attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints ONE JSON line.  `value` is the training-shape causal forward (B=32, H=12,
T=512, Dh=64, bf16 in / bf16 out, fp32 accumulate, SSMax on) in TFLOP/s, with one
step = one bam_attn_fwd call (at this shape one kernel, which computes its own bias)
on inputs already resident in HBM.  `parts` carries the other figures the metric names: the forward at
T=32768 (% of bf16 MFMA peak), decode against a 256,000-token KV cache (GB/s, % of
HBM peak) and the training-shape forward+backward.  FLOPs count 4*Dh per visible
causal (query, key) pair for the forward and 10*Dh for the backward; decode bytes are
the K and V bytes of the kv_len visible tokens.

`roofline` is for the dominant kernel of the `value` workload: its algorithmic bytes
per launch divided by its average launch duration, measured here with HIP events
around each launch on the stream it runs on.  `traffic` comes from the committed
rocprofv3 counter summary in profiles/, and is null when the kernel source has changed
since those counters were taken.  `cpu_baseline` is the fp64 oracle on this host's
cores (a process pool of single-threaded workers, one (b, h) head per task): `value` on
the training-shape forward in full, and per configuration in `configs` (the backward and
the 256k decode in full, the 32k forward on a row sample).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "BAM attn fwd TFLOP/s @T=512 & 32k (% MFMA peak); decode GB/s @256k KV"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
COUNTERS = os.path.join(ROOT, "profiles", "fwd_bf16_kernel_T512_counters.json")
SPIN_CYCLES = 20_000_000    # about 8 ms of GPU clock: time for the host to queue the timed launches
FWD_SRC = os.path.join(ROOT, "positional_prior_bias_amd", "csrc", "fwd.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_flops(B, H, T, Dh, causal=True):
    pairs = T * (T + 1) // 2 if causal else T * T
    return 4.0 * Dh * B * H * pairs


def src_sha(path):
    """sha256[:16] of a kernel source's code: comments and blank lines are dropped first, so
    an edit to comments alone leaves the committed counter summary valid."""
    with open(path, encoding="utf-8") as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    lines = (re.sub(r"//.*", "", l).rstrip() for l in text.splitlines())
    code = "\n".join(l for l in lines if l.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


class Timer:
    """Whole-step timing (events at both ends of K steps) and per-launch event pairs."""

    def __init__(self, torch):
        self.torch = torch

    def steps(self, fn, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        return e0.elapsed_time(e1) / steps, wall

    def cold_launch(self, fn, reps):
        """Median duration of one launch right after a 1 GiB device write, which evicts the
        inputs from L2 and the 256 MB MALL (each launch timed alone with an event pair)."""
        torch = self.torch
        junk = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        times = []
        for _ in range(reps):
            junk.fill_(1)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        del junk
        return sorted(times)[len(times) // 2]

    def per_launch(self, fn, launches, warmup=2):
        """Average duration of one launch of `fn`'s kernel: one event pair around `launches`
        back-to-back launches on the stream the kernel runs on.  A bounded spin kernel
        (torch.cuda._sleep) runs first on that stream, so the host has queued every launch
        before the GPU reaches the first event: the pair then measures GPU time even where
        one Python call takes longer than one kernel."""
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        spin = getattr(torch.cuda, "_sleep", None)   # private torch API: without it the pair
        if spin is not None:                           # may include host launch time
            spin(SPIN_CYCLES)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(launches):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / launches


def device_inputs(torch, w, with_grad=False):
    def d(x, bf16=True):
        if isinstance(x, torch.Tensor):   # drawn on the device already
            return x
        t = torch.from_numpy(x)
        return (t.to(torch.bfloat16) if bf16 else t.to(torch.float32)).cuda()
    out = dict(q=d(w.q), k=d(w.k), v=d(w.v), alpha=d(w.alpha, False), beta=d(w.beta, False), mu=d(w.mu, False),
               s=d(w.s, False))
    if with_grad:
        out["do"] = d(w.do)
    return out


def bench_fwd(torch, bam, w, steps, warmup, timer, name, cold=False):
    x = device_inputs(torch, w)
    B, H, T, Dh = w.q.shape
    o = torch.empty((B, H, T, Dh), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    ws = torch.empty(bam.bam_fwd_workspace_size(B, H, T, Dh, 3), dtype=torch.uint8, device="cuda")

    def call(table_ready=False):
        bam.bam_attn_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["mu"], x["s"], causal=True, ssmax=True,
                         o=o, lse=lse, workspace=ws, table_ready=table_ready)
    ms, wall = timer.steps(call, steps, warmup)
    kern_ms = timer.per_launch(lambda: call(True), max(steps, 10))
    cold_ms = timer.cold_launch(lambda: call(True), 10) if cold else None
    flops = fwd_flops(B, H, T, Dh)
    algo_bytes = 4 * B * H * T * Dh * 2 + B * H * T * 4   # Q, K, V read + O write (bf16) + lse
    log(f"[{name}] step {ms:.4f} ms (wall {wall:.4f}), fwd kernel {kern_ms:.4f} ms")
    if cold_ms is not None:
        log(f"[{name}] cold fwd kernel (caches flushed by a 1 GiB write) {cold_ms:.4f} ms")
    return dict(ms=ms, wall_ms=wall, kernel_ms=kern_ms, cold_kernel_ms=cold_ms, flops=flops, bytes=algo_bytes,
                tflops=flops / ms / 1e9, kernel_tflops=flops / kern_ms / 1e9,
                kernel_gbs=algo_bytes / kern_ms / 1e6)


def bench_skip(torch, bam, w, steps, timer):
    """Prior-aware key skipping (BAM_SKIP_FAR) on the 32k prefill: the forward call with and
    without it, table prebuilt in both (the skipping plan's kernels are inside the timed
    call).  Two prior settings: the workload's own heads, and the pages' AttentionPrior
    initialisation in the reference form (theta_alpha = ALiBi slopes, theta_beta =
    linspace(0, 1), theta_mu = 0, s = 1 / ln 512).  The backward call with and without
    skipping as well.  Skipping changes the work, not the result, so these figures are kept
    apart from the algorithmic-flop metric."""
    x = device_inputs(torch, w)
    B, H, T, Dh = w.q.shape
    o = torch.empty((B, H, T, Dh), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    slopes = bam.alibi_slopes(H, device="cuda")
    init = dict(alpha=slopes, beta=torch.linspace(0, 1, H, dtype=torch.float32, device="cuda"),
                mu=torch.zeros(H, dtype=torch.float32, device="cuda"),
                s=torch.full((H,), 1.0 / math.log(512.0), dtype=torch.float32, device="cuda"))
    out = {}
    for name, p, ref in (("workload_heads", x, False), ("pages_init_ref_form", init, True)):
        flags = bam.BAM_CAUSAL | bam.BAM_SSMAX | bam.BAM_SKIP_FAR | (bam.BAM_PRIOR_REF if ref else 0)
        ws = torch.empty(bam.bam_fwd_workspace_size(B, H, T, Dh, flags), dtype=torch.uint8, device="cuda")

        def call(skip, table_ready=True):
            bam.bam_attn_fwd(x["q"], x["k"], x["v"], p["alpha"], p["beta"], p["mu"], p["s"], causal=True,
                             ssmax=True, o=o, lse=lse, workspace=ws, table_ready=table_ready, prior_ref=ref,
                             skip_far=skip)
        call(True, table_ready=False)
        frac = bam.fwd_skipped_fraction(ws, B, H, T, Dh, flags)
        full = timer.per_launch(lambda: call(False), steps)
        skip = timer.per_launch(lambda: call(True), steps)
        flops = fwd_flops(B, H, T, Dh)
        log(f"[skip32k:{name}] full {full:.4f} ms, skipping {skip:.4f} ms, skipped fraction {frac:.3f}")
        out[name] = {"skipped_tile_fraction": round(frac, 4), "full_ms": round(full, 4), "skip_ms": round(skip, 4),
                     "speedup": round(full / skip, 3),
                     "effective_TFLOP/s": round(flops / skip / 1e9, 1)}
        # the backward call with and without skipping (its own plan over 128-query blocks
        # inside the timed call), gradients for every input and parameter
        call(False)
        dout = torch.randn((B, H, T, Dh), generator=torch.Generator(device="cuda").manual_seed(2), device="cuda",
                           dtype=torch.float32).to(torch.bfloat16)
        wsb = torch.empty(bam.bam_bwd_workspace_size(B, H, T, Dh, flags), dtype=torch.uint8, device="cuda")

        def bwd(skip_far):
            bam.bam_attn_bwd_ex(x["q"], x["k"], x["v"], o, lse, dout, p["alpha"], p["beta"], p["mu"], p["s"],
                                causal=True, ssmax=True, workspace=wsb, prior_ref=ref, skip_far=skip_far)
        bfull = timer.per_launch(lambda: bwd(False), max(2, steps // 2))
        bskip = timer.per_launch(lambda: bwd(True), max(2, steps // 2))
        log(f"[skip32k:{name}] backward full {bfull:.4f} ms, skipping {bskip:.4f} ms")
        out[name].update({"bwd_full_ms": round(bfull, 4), "bwd_skip_ms": round(bskip, 4),
                          "bwd_speedup": round(bfull / bskip, 3)})
    return out


def bench_fwdbwd(torch, bam, w, steps, warmup, timer):
    x = device_inputs(torch, w, with_grad=True)
    B, H, T, Dh = w.q.shape
    o = torch.empty((B, H, T, Dh), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    wsf = torch.empty(bam.bam_fwd_workspace_size(B, H, T, Dh, 3), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(bam.bam_bwd_workspace_size(B, H, T, Dh, 3), dtype=torch.uint8, device="cuda")

    def fwd():
        bam.bam_attn_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["mu"], x["s"], causal=True, ssmax=True,
                         o=o, lse=lse, workspace=wsf)

    def bwd():
        bam.bam_attn_bwd(x["q"], x["k"], x["v"], o, lse, x["do"], x["alpha"], x["beta"], x["mu"], x["s"],
                         causal=True, ssmax=True, workspace=wsb)

    def step():
        fwd()
        bwd()
    ms, wall = timer.steps(step, steps, warmup)
    bwd_ms = timer.per_launch(bwd, max(steps, 10))
    pairs = B * H * T * (T + 1) // 2
    flops = 14.0 * Dh * pairs
    # algorithmic bytes of one backward call: Q, K, V, O, dO read and dQ, dK, dV written
    # (bf16, 2 B per element each), lse read (4 B per row); the tables and per-row scalars
    # (under 1% of it) are left out
    bwd_bytes = 8 * B * H * T * Dh * 2 + B * H * T * 4
    log(f"[fwdbwd512] step {ms:.4f} ms, bwd call {bwd_ms:.4f} ms")
    return dict(ms=ms, wall_ms=wall, bwd_call_ms=bwd_ms, flops=flops, tflops=flops / ms / 1e9,
                bwd_tflops=10.0 * Dh * pairs / bwd_ms / 1e9, bwd_bytes=bwd_bytes,
                bwd_gbs=bwd_bytes / bwd_ms / 1e6)


def bench_decode(torch, bam, w, steps, warmup, timer):
    B, H, L, Dh = w.k.shape
    q = torch.from_numpy(w.q).to(torch.bfloat16).cuda()
    k, v = w.k, w.v     # already on the device (long_decode_device)
    kv = torch.from_numpy(w.kv_len).cuda()
    p = {n: torch.from_numpy(getattr(w, n)).cuda() for n in ("alpha", "beta", "mu", "s")}
    o = torch.empty((B, H, Dh), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(bam.bam_decode_workspace_size(B, H, L, Dh), dtype=torch.uint8, device="cuda")

    def call(table_ready=False):
        bam.bam_attn_decode(q, k, v, kv, p["alpha"], p["beta"], p["mu"], p["s"], ssmax=True, o=o, lse=lse,
                            workspace=ws, table_ready=table_ready)
    ms, wall = timer.steps(call, steps, warmup)
    kern_ms = timer.per_launch(lambda: call(True), max(steps, 10))
    nbytes = 2.0 * float(w.kv_len.astype("int64").sum()) * H * Dh * 2
    log(f"[decode] step {ms:.4f} ms, split+combine {kern_ms:.4f} ms")
    return dict(ms=ms, wall_ms=wall, kernels_ms=kern_ms, bytes=nbytes, gbs=nbytes / ms / 1e6,
                kernels_gbs=nbytes / kern_ms / 1e6)


def bench_decode_skip(torch, bam, w, steps, timer, full_kernels_ms):
    """Prior-aware decode skipping on the same workload: the key-norm pages (built once per
    cache change), the skipping call's kernels with the table prebuilt (bound + split +
    combine), the fraction of key ranges left out, and whether the output has the full
    call's bits."""
    B, H, L, Dh = w.k.shape
    q = torch.from_numpy(w.q).to(torch.bfloat16).cuda()
    kv = torch.from_numpy(w.kv_len).cuda()
    p = {n: torch.from_numpy(getattr(w, n)).cuda() for n in ("alpha", "beta", "mu", "s")}
    ws = torch.empty(bam.bam_decode_workspace_size(B, H, L, Dh), dtype=torch.uint8, device="cuda")
    norms = torch.empty((B, H, bam.bam_decode_norm_pages(L)), dtype=torch.float32, device="cuda")
    norms_ms = timer.per_launch(lambda: bam.bam_decode_key_norms(w.k, norms=norms), 10)
    o_full, l_full = bam.bam_attn_decode(q, w.k, w.v, kv, p["alpha"], p["beta"], p["mu"], p["s"], ssmax=True,
                                         o_dtype=torch.float32, workspace=ws)
    o_full, l_full = o_full.clone(), l_full.clone()
    o = torch.empty((B, H, Dh), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")

    def call(table_ready=True):
        bam.bam_attn_decode_skip(q, w.k, w.v, kv, p["alpha"], p["beta"], p["mu"], p["s"], key_norms=norms, ssmax=True,
                                 o=o, lse=lse, workspace=ws, table_ready=table_ready)
    call(False)
    torch.cuda.synchronize()
    same = bool(torch.equal(o.view(torch.int32), o_full.view(torch.int32)) and
                torch.equal(lse.view(torch.int32), l_full.view(torch.int32)))
    frac = bam.decode_skipped_fraction(ws, kv, B, H, L, Dh)
    kern_ms = timer.per_launch(call, max(steps, 10))
    nbytes = 2.0 * float(w.kv_len.astype("int64").sum()) * H * Dh * 2
    log(f"[decode skip] ranges skipped {frac:.3f}, kernels {kern_ms:.4f} ms (full {full_kernels_ms:.4f}), "
        f"norm pages {norms_ms:.4f} ms, same bits {same}")
    return {"note": "prior-aware decode skipping: the same bits as the full call, less work; effective_GB/s = the "
                    "dense K+V bytes / the skipping kernels' time, not the metric",
            "skipped_range_fraction": round(frac, 4), "same_bits_as_full": same,
            "full_kernels_ms": round(full_kernels_ms, 4), "skip_kernels_ms": round(kern_ms, 4),
            "speedup": round(full_kernels_ms / kern_ms, 3), "effective_GB/s": round(nbytes / kern_ms / 1e6, 1),
            "key_norm_pages_ms": round(norms_ms, 4)}


def bench_train_step(torch, w, steps, warmup, timer):
    """Forward + backward through the autograd module (reference parameterisation, every
    prior parameter trained, SSMax on), gradients for q, k, v and the prior."""
    from positional_prior_bias_amd.autograd import BamAttention
    m = BamAttention(w.q.shape[1], max_seq_len=w.q.shape[2], train_theta_mu=True, device="cuda")
    x = device_inputs(torch, w, with_grad=True)
    q, k, v = (x[n].requires_grad_(True) for n in ("q", "k", "v"))
    do = x["do"]

    def step():
        for t in [q, k, v] + list(m.parameters()):
            t.grad = None
        o = m(q, k, v)
        o.backward(do)
    # The backward on the calling thread: with the engine's per-device worker thread the
    # step's host side (two thread hand-offs per backward) outlasts its GPU work.
    with torch.autograd.set_multithreading_enabled(False):
        ms, wall = timer.steps(step, steps, warmup)
    ms_mt, wall_mt = timer.steps(step, steps, warmup)
    log(f"[train512] step {ms:.4f} ms (wall {wall:.4f}); with the engine's worker thread {ms_mt:.4f} ms")
    return dict(ms=ms, wall_ms=wall, autograd="backward on the calling thread (set_multithreading_enabled(False))",
                ms_engine_worker_thread=ms_mt)


def bench_sweep(torch, bam, wl, timer):
    """Passkey-style length sweep: causal prefill at T = 1k .. 262k (32,768 tokens per batch
    up to 32k, then B = 1) and decode against caches of 4k .. 512k tokens (B = 8, one planted
    key per sequence).  Inputs from 64k on are drawn on the device."""
    out = {"prefill": [], "decode": []}
    for T in (1024, 4096, 16384, 32768, 65536, 131072, 262144):
        B = max(1, 32768 // T)
        w = wl.long_prefill(T=T, B=B) if T <= 32768 else wl.long_prefill_device(T=T, B=B)
        r = bench_fwd(torch, bam, w, 3, 1, timer, f"sweep fwd T={T}")
        out["prefill"].append({"T": T, "B": B, "kernel_ms": round(r["kernel_ms"], 4),
                               "kernel_TFLOP/s": round(r["kernel_tflops"], 1),
                               "kernel_pct_mfma_peak": round(100 * r["kernel_tflops"] / PEAK_BF16_TFLOPS, 2),
                               "step_TFLOP/s": round(r["tflops"], 1)})
        del w
        torch.cuda.empty_cache()
    for L in (4096, 32768, 131072, 262144, 524288):
        w = wl.long_decode_device(L=L)
        r = bench_decode(torch, bam, w, 5, 2, timer)
        out["decode"].append({"L": L, "step_ms": round(r["ms"], 4), "step_GB/s": round(r["gbs"], 1),
                              "kernels_GB/s": round(r["kernels_gbs"], 1)})
        del w
        torch.cuda.empty_cache()
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host cores, one (b, h) unit per task in a process
# pool whose workers run single-threaded BLAS.  The pool is started before the GPU is
# touched and stays idle while the GPU parts run; each CPU leg runs right after its GPU part.
# ---------------------------------------------------------------------------------------

_SINGLE_THREAD_ENV = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")


def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass
    import oracle  # noqa: F401  (import cost paid before any task is timed)


def _cpu_noop(_):
    time.sleep(0.05)   # long enough that every worker takes one
    return os.getpid()


def _cpu_task(task):
    """One (b, h) unit of the oracle: ("fwd" | "fwdbwd" | "rows" | "decode", arrays...)."""
    import numpy as np
    import oracle
    kind = task[0]
    if kind == "fwd":
        _, q, k, v, a, b, m, s = task
        oracle.attn_fwd(q[None, None], k[None, None], v[None, None], [a], [b], [m], [s], causal=True, ssmax=True)
    elif kind == "fwdbwd":
        _, q, k, v, do, a, b, m, s = task
        oracle.attn_fwd(q[None, None], k[None, None], v[None, None], [a], [b], [m], [s], causal=True, ssmax=True)
        oracle.attn_bwd(q[None, None], k[None, None], v[None, None], do[None, None], [a], [b], [m], [s],
                        causal=True, ssmax=True)
    elif kind == "rows":
        _, q, k, v, rows, a, b, m, s = task
        oracle.attn_fwd_rows(q, k, v, rows, a, b, m, s, causal=True, ssmax=True)
    elif kind == "decode":
        _, q, kbits, vbits, n, a, b, m, s = task
        widen = lambda x: (x.astype(np.uint32) << 16).view(np.float32)  # noqa: E731  (bf16 bits)
        oracle.attn_decode(q[None, None], widen(kbits)[None, None], widen(vbits)[None, None], [n], [a], [b], [m],
                           [s], ssmax=True)
    return os.getpid()


class CpuOracle:
    """The process pool and the per-configuration oracle timings."""

    def __init__(self, seconds):
        import multiprocessing as mp
        self.cores = max(1, min(16, len(os.sched_getaffinity(0))))
        self.seconds = seconds
        saved = {k: os.environ.get(k) for k in _SINGLE_THREAD_ENV}
        for k in _SINGLE_THREAD_ENV:
            os.environ[k] = "1"
        try:
            self.pool = mp.get_context("spawn").Pool(self.cores, initializer=_cpu_worker_init)
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
        self.pool.map(_cpu_noop, range(2 * self.cores), chunksize=1)
        self.used = set()   # worker processes that ran timed tasks
        self.results = {}

    @property
    def workers(self):
        return len(self.used) if self.used else self.cores

    def close(self):
        self.pool.close()
        self.pool.join()

    def _run(self, tasks):
        t0 = time.perf_counter()
        for pid in self.pool.imap_unordered(_cpu_task, tasks):
            self.used.add(pid)
        return time.perf_counter() - t0

    def _passes(self, make_tasks):
        """Whole passes over the batch until `seconds` have elapsed (at least one)."""
        el, n = 0.0, 0
        while n == 0 or el < self.seconds:
            el += self._run(make_tasks())
            n += 1
        return el, n

    def fwd_full(self, w):
        B, H, T, Dh = w.q.shape
        mk = lambda: [("fwd", w.q[b, h], w.k[b, h], w.v[b, h], w.alpha[h], w.beta[h], w.mu[h], w.s[h])  # noqa: E731
                      for b in range(B) for h in range(H)]
        el, n = self._passes(mk)
        flops = n * fwd_flops(B, H, T, Dh)
        self.results["fwd_T512"] = {
            "workload": f"causal fwd B={B} H={H} T={T} Dh={Dh}, every row", "passes": n, "seconds": round(el, 2),
            "TFLOP/s": flops / el / 1e12}
        return self.results["fwd_T512"]

    def fwdbwd_full(self, w):
        B, H, T, Dh = w.q.shape
        mk = lambda: [("fwdbwd", w.q[b, h], w.k[b, h], w.v[b, h], w.do[b, h], w.alpha[h], w.beta[h], w.mu[h],  # noqa: E731
                       w.s[h]) for b in range(B) for h in range(H)]
        el, n = self._passes(mk)
        flops = n * 14.0 * Dh * B * H * T * (T + 1) / 2
        self.results["fwd_bwd_T512"] = {
            "workload": f"causal fwd+bwd B={B} H={H} T={T} Dh={Dh}, every row", "passes": n,
            "seconds": round(el, 2), "TFLOP/s": flops / el / 1e12}

    def rows_sample(self, w, nrows=256, seed=0):
        """The T = 32768 forward on a stratified row sample: nrows rows per head, evenly
        spread over [0, T) (each row costs keys 0..i), extrapolated to every row by the
        visible-pair count."""
        import numpy as np
        B, H, T, Dh = w.q.shape
        rows = np.unique(np.linspace(0, T - 1, nrows).round().astype(np.int64))
        tasks = [("rows", w.q[0, h], w.k[0, h], w.v[0, h], rows, w.alpha[h], w.beta[h], w.mu[h], w.s[h])
                 for h in range(H)]
        el = self._run(tasks)
        pairs_sampled = float(H * (rows + 1).sum())
        rate = 4.0 * Dh * pairs_sampled / el
        self.results["fwd_T32768"] = {
            "workload": f"causal fwd B={B} H={H} T={T} Dh={Dh}: {rows.size} rows per head sampled evenly over [0, T)",
            "seconds": round(el, 2), "TFLOP/s": rate / 1e12,
            "extrapolated_full_call_s": round(fwd_flops(B, H, T, Dh) / rate, 1),
            "note": "rate measured on the sampled rows; the full-call time is extrapolated by visible pairs"}

    def decode_full(self, w):
        """Every (b, h) of the 256,000-token decode: each slab is copied to the host (bf16 bits)
        and sent to a worker; the copy runs while the pool computes earlier slabs."""
        import numpy as np
        import torch
        B, H, L, Dh = w.k.shape

        def tasks():
            for b in range(B):
                n = int(w.kv_len[b])
                for h in range(H):
                    kb = w.k[b, h, :n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                    vb = w.v[b, h, :n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                    yield ("decode", w.q[b, h], kb, vb, n, w.alpha[h], w.beta[h], w.mu[h], w.s[h])
        el = self._run(tasks())
        nbytes = 2.0 * float(w.kv_len.astype("int64").sum()) * H * Dh * 2
        self.results["decode_256k"] = {
            "workload": f"decode B={B} H={H} L={L} Dh={Dh}, every (b, h), bf16 cache widened on the host",
            "seconds": round(el, 2), "GB/s": nbytes / el / 1e9,
            "note": "includes the device-to-host copy of each K/V slab, overlapped with the pool's work"}

    def summary(self):
        r = self.results.get("fwd_T512")
        if r is None:
            return None
        return {"value": r["TFLOP/s"], "unit": "TFLOP/s", "cores": self.workers, "kind": "oracle",
                "sample": f"the training-shape forward in full ({r['workload']}), {r['passes']} passes in "
                          f"{r['seconds']} s: a spawn process pool of {self.workers} workers, one (b, h) head per "
                          f"task, single-threaded fp64 numpy each, on {_cpu_model()}; per-configuration figures "
                          f"in configs",
                "configs": {k: {kk: (round(vv, 6) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                            for k, v in self.results.items()}}


def traffic_from_counters():
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None, "no counter summary"
    if c.get("source_sha") != src_sha(FWD_SRC):
        return None, "kernel changed since the counters were taken"
    return c.get("traffic_bytes"), c.get("command")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--parts", default="fwd512,fwd32k,skip32k,decode,fwdbwd512,train512,sweep",
                    help="comma list of fwd512,fwd32k,skip32k,decode,fwdbwd512,train512,sweep,cold512 (fwd512 is "
                         "always run; skip32k needs fwd32k; cold512, the T = 512 forward after a cache flush, "
                         "is not run by default so that every default launch of that kernel is a warm one)")
    ap.add_argument("--cpu-seconds", type=float, default=3.0,
                    help="minimum time of each whole-batch CPU-baseline leg (the batch is repeated)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for scaling HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (BAM attention shards with no "
              "exchange over heads/batch; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    parts = set(args.parts.split(",")) | {"fwd512"}
    # the CPU baseline's worker pool starts before anything touches the GPU
    cpu = None if args.no_cpu_baseline else CpuOracle(args.cpu_seconds)
    if cpu is not None:
        log(f"[cpu_baseline] pool of {cpu.workers} single-threaded workers on {_cpu_model()}")

    import numpy as np  # noqa: F401
    import torch

    import positional_prior_bias_amd as bam
    from positional_prior_bias_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    bam.lib()
    timer = Timer(torch)

    log("[fwd512] generating inputs")
    w2 = wl.training_shape()
    r512 = bench_fwd(torch, bam, w2, args.steps, args.warmup, timer, "fwd512", cold="cold512" in parts)
    out_parts = {"fwd_T512": {
        "workload": "causal fwd B=32 H=12 T=512 Dh=64 bf16, SSMax on",
        "ms": round(r512["ms"], 5), "TFLOP/s": round(r512["tflops"], 2),
        "pct_mfma_peak": round(100 * r512["tflops"] / PEAK_BF16_TFLOPS, 2),
        "kernel_ms": round(r512["kernel_ms"], 5), "kernel_TFLOP/s": round(r512["kernel_tflops"], 2),
        "kernel_algorithmic_GB/s": round(r512["kernel_gbs"], 1),
        "pct_hbm_peak": round(100 * r512["kernel_gbs"] / PEAK_HBM_GBS, 2)}}
    if r512["cold_kernel_ms"] is not None:
        out_parts["fwd_T512"]["cold_kernel_ms"] = round(r512["cold_kernel_ms"], 5)
        out_parts["fwd_T512"]["cold_kernel_TFLOP/s"] = round(r512["flops"] / r512["cold_kernel_ms"] / 1e9, 2)
    if cpu is not None:
        log("[cpu_baseline] training-shape forward")
        cpu.fwd_full(w2)

    if "fwd32k" in parts:
        log("[fwd32k] generating inputs")
        w4 = wl.long_prefill()
        r = bench_fwd(torch, bam, w4, max(3, args.steps // 4), 2, timer, "fwd32k")
        out_parts["fwd_T32768"] = {
            "workload": "causal fwd B=1 H=12 T=32768 Dh=64 bf16, 6 heavy-tailed + 6 inverted-prior heads, SSMax on",
            "ms": round(r["ms"], 4), "TFLOP/s": round(r["tflops"], 1),
            "pct_mfma_peak": round(100 * r["tflops"] / PEAK_BF16_TFLOPS, 2),
            "kernel_ms": round(r["kernel_ms"], 4), "kernel_TFLOP/s": round(r["kernel_tflops"], 1),
            "kernel_pct_mfma_peak": round(100 * r["kernel_tflops"] / PEAK_BF16_TFLOPS, 2),
            "roofline": {"bound": "mfma", "achieved": round(r["kernel_tflops"], 1), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(r["kernel_tflops"] / PEAK_BF16_TFLOPS, 4)}}
        if "skip32k" in parts:
            out_parts["skip_T32768"] = {
                "note": "prior-aware key skipping: same results, less work; effective_TFLOP/s = the dense "
                        "algorithmic flops / the skipping call's time, not the metric",
                **bench_skip(torch, bam, w4, max(3, args.steps // 4), timer)}
        if cpu is not None:
            log("[cpu_baseline] 32k forward, row sample")
            cpu.rows_sample(w4)
        del w4
    if "decode" in parts:
        log("[decode] generating inputs (256,000-token caches)")
        w5 = wl.long_decode_device()
        r = bench_decode(torch, bam, w5, max(5, args.steps // 2), 3, timer)
        out_parts["decode_256k"] = {
            "workload": "decode B=8 H=12 Dh=64, bf16 KV cache of 256,000 tokens, one planted key per sequence",
            "ms": round(r["ms"], 4), "GB/s": round(r["gbs"], 1), "pct_hbm_peak": round(100 * r["gbs"] / PEAK_HBM_GBS, 2),
            "kernels_ms": round(r["kernels_ms"], 4),
            "roofline": {"bound": "hbm", "achieved": round(r["kernels_gbs"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(r["kernels_gbs"] / PEAK_HBM_GBS, 4),
                         "note": "split + combine kernels (table prebuilt), K+V bytes of the visible tokens"}}
        out_parts["decode_256k"]["skip"] = bench_decode_skip(torch, bam, w5, max(5, args.steps // 2), timer,
                                                             r["kernels_ms"])
        if cpu is not None:
            log("[cpu_baseline] 256k decode, every (b, h)")
            cpu.decode_full(w5)
        del w5
        torch.cuda.empty_cache()
    if "fwdbwd512" in parts:
        log("[fwdbwd512] generating inputs")
        w3 = wl.training_shape(with_grad=True)
        r = bench_fwdbwd(torch, bam, w3, args.steps, args.warmup, timer)
        out_parts["fwd_bwd_T512"] = {
            "workload": "causal fwd+bwd B=32 H=12 T=512 Dh=64 bf16, dQ/dK/dV bf16 + per-head dalpha/dbeta/ds",
            "ms": round(r["ms"], 4), "TFLOP/s": round(r["tflops"], 1),
            "pct_mfma_peak": round(100 * r["tflops"] / PEAK_BF16_TFLOPS, 2),
            "bwd_call_ms": round(r["bwd_call_ms"], 4), "bwd_TFLOP/s": round(r["bwd_tflops"], 1),
            "bwd_roofline": {"bound": "hbm", "achieved": round(r["bwd_gbs"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(r["bwd_gbs"] / PEAK_HBM_GBS, 4),
                             "algorithmic_bytes_per_call": r["bwd_bytes"],
                             "pct_mfma_peak": round(100 * r["bwd_tflops"] / PEAK_BF16_TFLOPS, 2),
                             "note": "whole backward call (bwd_dq + bwd_dkdv; no table launch at T <= 512): "
                                     "Q, K, V, O, dO read, dQ, dK, dV written (bf16) and lse read"}}
        if "train512" in parts:
            r = bench_train_step(torch, w3, args.steps, args.warmup, timer)
            out_parts["train_step_T512"] = {
                "workload": "autograd step through BamAttention at B=32 H=12 T=512 Dh=64: forward + backward, "
                            "grads for q, k, v, theta_alpha, theta_beta, theta_mu, s",
                "ms": round(r["ms"], 4), "wall_ms": round(r["wall_ms"], 4),
                "TFLOP/s": round(14.0 * 64 * 32 * 12 * 512 * 513 / 2 / r["ms"] / 1e9, 1),
                "autograd": r["autograd"], "ms_engine_worker_thread": round(r["ms_engine_worker_thread"], 4)}
        if cpu is not None:
            log("[cpu_baseline] training-shape forward + backward")
            cpu.fwdbwd_full(w3)
        del w3

    if "sweep" in parts:
        out_parts["length_sweep"] = bench_sweep(torch, bam, wl, timer)

    if args.copy_calibration:
        n = 512 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[copy-calibration] copied {n} bytes 3 times")

    traffic, tnote = traffic_from_counters()
    roof = {"bound": "hbm", "achieved": round(r512["kernel_gbs"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(r512["kernel_gbs"] / PEAK_HBM_GBS, 4), "traffic": traffic,
            "kernel": "fwd_bf16_kernel<64,causal>",
            "algorithmic_bytes_per_launch": r512["bytes"],
            "kernel_ms": round(r512["kernel_ms"], 5)}
    if traffic is None:
        roof["traffic_note"] = tnote

    cpu_line = None
    if cpu is not None:
        cpu_line = cpu.summary()
        cpu.close()
        gpu = {"fwd_T512": out_parts["fwd_T512"].get("kernel_TFLOP/s"),
               "fwd_T32768": out_parts.get("fwd_T32768", {}).get("kernel_TFLOP/s"),
               "fwd_bwd_T512": out_parts.get("fwd_bwd_T512", {}).get("TFLOP/s"),
               "decode_256k": out_parts.get("decode_256k", {}).get("GB/s")}
        for k, v in cpu_line["configs"].items():
            g = gpu.get(k)
            c = v.get("TFLOP/s", v.get("GB/s"))
            if g and c:
                v["gpu_over_cpu"] = round(g / c, 1)

    line = {
        "metric": METRIC, "value": round(r512["tflops"], 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r512["ms"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, per-head prior parameters as documented)",
        "config": {"workload": "training-shape causal BAM attention forward, B=32 H=12 T=512 Dh=64, bf16 in/out, "
                               "fp32 accumulate, SSMax on; one step = bam_attn_fwd (one kernel: it computes its own bias)",
                   "B": 32, "H": 12, "T": 512, "Dh": 64, "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu_line, "parts": out_parts,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
