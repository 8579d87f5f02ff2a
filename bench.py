#!/usr/bin/env python3
"""Throughput of Positional-LSH ALiBi attention on one MI355X.

A step is one pass of the whole path over one batch of resident inputs,
one plpsh_attention_fwd call: host draw of the s hashes per head, then one
kernel that evaluates the bins of each query tile, writes the bin buffer
(block counts, block starts, plan records) and computes the count-weighted
attention.  Default workload: one Mistral-7B-shaped
attention layer (batch 1, 32 query / 8 KV heads, n = 16384, head_dim 128,
bf16, causal, s = 20, sigma_h = 2^(8(h+1)/32)), synthetic N(0, 1) inputs.

The timed loop (`value`, `ms_per_step`: W untimed warmup steps, then K
timed steps between two synchronisations) records nothing but the steps.
Separate passes before it, on the same buffers, give the per-step
distribution (one event per step boundary) and the attention kernel's
duration (an event pair around each launch, on the stream it runs on).

Prints ONE JSON line.  Besides the contract fields it carries:
  step_ms      : median, p10, p90 of the step time (separate pass: 20
                 groups of 5 steps, an event at each group boundary)
  two_launch   : the same step as two launches (plpsh_sample_bins, whose
                 bin kernel writes the buffer, then plpsh_attention_fwd_bins)
  roofline     : the step's kernel against the HBM roofline: algorithmic
                 bytes (Q, K, V read once + O and the bin buffer written
                 once, per launch)
                 divided by the kernel's median duration with the L2 and the
                 last-level cache evicted (by a read-only pass over 512 MiB)
                 before each launch (the roofline
                 figure: a step's inputs are not cache-resident in a model);
                 the back-to-back (warm-cache) figures side by side
  workloads    : tiny, small, qwen3, long: tokens/s of the step, the
                 kernel's cold- and warm-cache median, cold-cache HBM fraction
  cpu_baseline : the fp64 oracle timed on a bounded sample of the same
                 workload by a pool of worker processes (one per core of the
                 host's share, one BLAS thread each)
  dense_alibi  : exact ALiBi (plpsh_alibi_dense_fwd) at the same n
  literal      : the same step with the attention computed as one short
                 attention per hash (plpsh_attention_fwd_literal, the
                 reduction of Theorem 2.2 taken literally), same bins
  backward     : a training step's attention on the same bins: the forward
                 with row normalisers (plpsh_attention_fwd_lse) and the
                 backward pass (plpsh_attention_bwd), each timed with HIP
                 events over 30 steps after 10 untimed ones (medians, and
                 the backward's p10 / p90); useful MFMA rate of the backward
                 (5 products per counted pair against the forward's 2)
  fixed_blocks : the deterministic fixed-blocks baseline (plpsh_fixed_blocks_fwd,
                 block b_h = round(2 sigma_h), the mean of Gamma(2, sigma_h))
  crossover    : PLSH vs dense ALiBi step times over n = 512 .. 131072
                 (Mistral shape, s = 20)
  long_context : the long-context workload (n = 131072, s = 32) as a step,
                 against dense ALiBi at the same n
  convergence  : ||L* - M~||_2 and ||L* - M~||_max against s at n = 131072,
                 sigma = 256 (plpsh_error_norms), with the fitted log-log
                 slopes and the time per measurement
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "approx-ALiBi attn tokens/s + % MFMA/HBM roofline, n=16k s=20 Mistral-7B shape"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "plsh_fwd_mistral_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "randomized_positional_lsh_amd", "csrc", "attn.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def algorithmic_bytes(W) -> int:
    """Q, K, V read once and O written once (bytes per launch)."""
    eb = 2 if W.dtype == "bf16" else 4
    return eb * W.batch * W.n * W.head_dim * (2 * W.heads_q + 2 * W.heads_kv)


def bin_buffer_bytes(W, P, ws) -> int:
    """Bytes of the bin buffer that the one-launch kernel writes besides O:
    the block counts, every block start with its closing entry n (counted
    from the counts of this draw), and the plan records."""
    nblk = P.Bins(ws, W.heads_q, W.s, W.n).nblk.cpu().numpy().astype(int)
    ntile = (W.n + 127) // 128
    return 4 * nblk.size + 4 * int((nblk + 1).sum()) + 32 * W.heads_q * ntile * W.s


def useful_flops(W, P, ws) -> float:
    """4 d per (row, key) pair inside the row's support [lo(r), hi(r)) (cut
    at r + 1 when causal), counted exactly from the block starts the bin
    kernel wrote for this draw: the least work that yields the output."""
    import numpy as np
    bins = P.Bins(ws, W.heads_q, W.s, W.n)
    nblk = bins.nblk.cpu().numpy()
    starts = bins.starts.cpu().numpy()
    rows = np.arange(W.n)
    tot = 0
    for h in range(W.heads_q):
        lo = np.full(W.n, W.n, dtype=np.int64)
        hi = np.zeros(W.n, dtype=np.int64)
        for i in range(W.s):
            t = h * W.s + i
            st = starts[t, :nblk[t] + 1].astype(np.int64)
            kb = np.searchsorted(st, rows, side="right") - 1
            lo = np.minimum(lo, st[kb])
            hi = np.maximum(hi, st[kb + 1])
        if W.causal:
            hi = np.minimum(hi, rows + 1)
        tot += int((hi - lo).sum())
    return 4.0 * W.head_dim * W.batch * tot


class Runner:
    """One step of the whole path with pre-marshalled C arguments."""

    def __init__(self, P, W, q, k, v, o, dev):
        import numpy as np
        import torch
        self.P, self.W = P, W
        self.lib = P.raw()
        self.sig = np.ascontiguousarray(W.sigmas, dtype=np.float64)
        self.delta = np.empty(W.heads_q * W.s)
        self.u = np.empty(W.heads_q * W.s)
        nb = P.bins_layout(W.heads_q, W.s, W.n)["total"]
        self.ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        self.q, self.k, self.v, self.o = q, k, v, o
        self.dtype = 1 if W.dtype == "bf16" else 0
        dp = ctypes.POINTER(ctypes.c_double)
        self.p_sig = self.sig.ctypes.data_as(dp)
        self.p_delta = self.delta.ctypes.data_as(dp)
        self.p_u = self.u.ctypes.data_as(dp)
        self.vp = [ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, o)]
        self.p_ws = ctypes.c_void_p(self.ws.data_ptr())
        self.nws = self.ws.numel()
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step(self):
        """The whole path in one call (one kernel launch)."""
        W = self.W
        st = self.lib.plpsh_attention_fwd(*self.vp, W.batch, W.heads_q, W.heads_kv, W.n, W.head_dim, self.dtype,
                                          self.p_sig, W.s, ctypes.c_uint64(W.hash_seed), int(W.causal), self.p_ws,
                                          self.nws, self.stream)
        if st:
            raise RuntimeError(self.P.status_string(st))

    def two_launch(self):
        """The same step as the bin kernel, then attention on its buffer."""
        self.bins()
        self.attn()

    def bins(self):
        W = self.W
        st = self.lib.plpsh_sample_bins(W.hash_seed, W.heads_q, W.s, W.n, self.p_sig, self.p_delta, self.p_u,
                                        self.p_ws, self.nws, self.stream)
        if st:
            raise RuntimeError(self.P.status_string(st))

    def attn_literal(self):
        W = self.W
        st = self.lib.plpsh_attention_fwd_literal(*self.vp, W.batch, W.heads_q, W.heads_kv, W.n, W.head_dim,
                                                  self.dtype, W.s, int(W.causal), self.p_ws, self.nws, self.p_delta,
                                                  self.stream)
        if st:
            raise RuntimeError(self.P.status_string(st))

    def attn(self):
        W = self.W
        st = self.lib.plpsh_attention_fwd_bins(*self.vp, W.batch, W.heads_q, W.heads_kv, W.n, W.head_dim, self.dtype,
                                               W.s, int(W.causal), self.p_ws, self.nws, self.p_delta, self.stream)
        if st:
            raise RuntimeError(self.P.status_string(st))


def time_steps(run, steps, warmup):
    """Wall time of `steps` back-to-back steps (nothing else is recorded on
    the stream in between)."""
    import torch
    for _ in range(warmup):
        run.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run.step()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def pct(x) -> dict:
    import numpy as np
    return {"median": round(float(np.median(x)), 5), "p10": round(float(np.percentile(x, 10)), 5),
            "p90": round(float(np.percentile(x, 90)), 5)}


def step_times(run, groups, per=5):
    """Step durations (ms), each the mean over a group of `per` consecutive
    steps between two events: an event on the stream holds it for several
    microseconds, which a group spreads over its steps."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(groups + 1)]
    ev[0].record()
    for i in range(groups):
        for _ in range(per):
            run.step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) / per for i in range(groups)]


def kernel_times(run, reps, cold):
    """Durations (ms) of the step's kernel, an event pair around each launch
    on its stream (the host draws the hashes while the GPU still runs the
    work enqueued before, so the pair spans the kernel).  cold: a 512 MiB buffer is
    read (summed) on the same stream before every launch, outside the events,
    which evicts the L2 and the 256 MB last-level cache; the eviction only
    reads, so no dirty lines of its own are written back during the launch.
    Untimed (eviction, launch) pairs come first: the first few dozen cold
    launches after warm work run slower while the device settles into the
    alternation (at the Mistral layer, whichever cold loop came first in a
    process measured 183-185 us per launch, every later one 170-171)."""
    import torch
    scratch = torch.ones(128 << 20, dtype=torch.float32, device=run.q.device) if cold else None
    for _ in range(100 if cold else 3):
        if scratch is not None:
            scratch.sum()
        run.step()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        if scratch is not None:
            scratch.sum()
        a.record()
        run.step()
        b.record()
    torch.cuda.synchronize()
    del scratch
    return [a.elapsed_time(b) for a, b in ev]


def _cpu_worker(job):
    """One worker of the CPU baseline: oracle tasks (64-row block, head) from
    the memory-mapped inputs, with one BLAS thread, from a common start time
    until `seconds` have passed."""
    import numpy as np
    import threadpoolctl
    threadpoolctl.threadpool_limits(1)
    import oracle
    d, tasks, causal, grp, seconds, t_start = job
    q = np.load(os.path.join(d, "q.npy"), mmap_mode="r")
    k = np.load(os.path.join(d, "k.npy"), mmap_mode="r")
    v = np.load(os.path.join(d, "v.npy"), mmap_mode="r")
    delta = np.load(os.path.join(d, "delta.npy"))
    u = np.load(os.path.join(d, "u.npy"))
    while time.time() < t_start:
        time.sleep(0.01)
    t0 = time.time()
    rows = done = 0
    for blk, h in tasks:
        out, _ = oracle.plsh_attention_rowblocks(q[h], k[h // grp], v[h // grp], delta[h], u[h], causal,
                                                 row_block=64, blocks=[blk])
        rows += out.shape[0]
        done += 1
        if time.time() - t0 >= seconds:
            break
    return rows, done, time.time() - t0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(W, q, k, v, delta, u, seconds):
    """The oracle, as it stands, on a bounded sample of the workload, by a
    pool of worker processes, one per core of the host's share (at most 16,
    the host share of one GPU), each with one BLAS thread: (64-row block,
    head) tasks, blocks in random order and every head per block (so every
    sigma is represented), dealt round-robin; every worker runs for `seconds`
    from a common start.  Workers are started fresh (spawn) and read the
    inputs from memory-mapped files."""
    import multiprocessing as mp
    import shutil
    import tempfile
    from concurrent.futures import ProcessPoolExecutor
    import numpy as np
    nproc = len(os.sched_getaffinity(0))
    workers = max(1, min(nproc, 16))
    d = tempfile.mkdtemp(prefix="plpsh_cpu_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        for name, t in (("q", q), ("k", k), ("v", v)):
            np.save(os.path.join(d, f"{name}.npy"), t[0].float().cpu().numpy())
        np.save(os.path.join(d, "delta.npy"), np.asarray(delta, dtype=np.float64))
        np.save(os.path.join(d, "u.npy"), np.asarray(u, dtype=np.float64))
        rng = np.random.default_rng(0)
        order = rng.permutation((W.n + 63) // 64)
        tasks = [(int(blk), h) for blk in order for h in range(W.heads_q)]
        grp = W.heads_q // W.heads_kv
        t_start = time.time() + 5.0  # after every worker has started and mapped its inputs
        jobs = [(d, tasks[i::workers], W.causal, grp, seconds, t_start) for i in range(workers)]
        # a worker that dies raises here (BrokenProcessPool) instead of hanging
        with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as pool:
            res = list(pool.map(_cpu_worker, jobs))
    finally:
        shutil.rmtree(d, ignore_errors=True)
    rows = sum(r[0] for r in res)
    done = sum(r[1] for r in res)
    el = max(r[2] for r in res)
    return {
        "value": rows / el / W.heads_q,  # a token needs one output row in every head
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "nproc": nproc,
        "cpu_model": cpu_model(),
        "sample": f"{done} (head, 64-row block) tasks = {rows} output rows over all {W.heads_q} heads in "
                  f"{el:.1f} s by {workers} worker processes with 1 BLAS thread each (banded fp64 oracle, "
                  f"hash seed {W.hash_seed})",
    }


def dense_alibi(P, W, q, k, v, steps=10, warmup=3):
    import torch
    o = torch.empty_like(q)
    for _ in range(warmup):
        P.alibi_dense(q, k, v, W.sigmas, causal=W.causal, out=o)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        P.alibi_dense(q, k, v, W.sigmas, causal=W.causal, out=o)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def literal(run, steps=10, warmup=3):
    """Mean duration (ms) of the per-hash attention kernel on the bins of
    the last timed step."""
    import torch
    for _ in range(warmup):
        run.attn_literal()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        run.attn_literal()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def backward(P, W, run, flops_fwd, steps=30, warmup=10):
    import numpy as np
    import torch
    q, k, v = run.q, run.k, run.v
    bins = P.Bins(run.ws, W.heads_q, W.s, W.n)
    delta = run.delta.reshape(W.heads_q, W.s)
    gen = torch.Generator(device=q.device)
    gen.manual_seed(9)
    do = torch.randn(q.shape, generator=gen, device=q.device, dtype=torch.float32).to(q.dtype)
    o = torch.empty_like(q)
    lse = torch.empty((W.batch, W.heads_q, W.n), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(P.raw().plpsh_attention_bwd_workspace_bytes(W.batch, W.heads_q, W.n), dtype=torch.uint8,
                     device=q.device)
    for _ in range(warmup):
        P.attention_lse(q, k, v, bins, causal=W.causal, delta=delta, out=o, lse=lse)
        P.attention_bwd(q, k, v, o, do, lse, bins, causal=W.causal, delta=delta, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for a, b, c in ev:
        a.record()
        P.attention_lse(q, k, v, bins, causal=W.causal, delta=delta, out=o, lse=lse)
        b.record()
        P.attention_bwd(q, k, v, o, do, lse, bins, causal=W.causal, delta=delta, dq=dq, dk=dk, dv=dv, workspace=ws)
        c.record()
    torch.cuda.synchronize()
    f_ms = float(np.median([a.elapsed_time(b) for a, b, _ in ev]))
    bt = np.array([b.elapsed_time(c) for _, b, c in ev])
    b_ms = float(np.median(bt))
    tflops = 2.5 * flops_fwd / (b_ms * 1e-3) / 1e12
    # algorithmic bytes: Q, O, dO, dQ (query-head sized), K, V, dK, dV (KV-head sized), LSE and D once each
    qsz = W.batch * W.heads_q * W.n * W.head_dim * 2
    kvsz = W.batch * W.heads_kv * W.n * W.head_dim * 2
    bwd_bytes = 4 * qsz + 4 * kvsz + 2 * 4 * W.batch * W.heads_q * W.n
    gbs = bwd_bytes / (b_ms * 1e-3) / 1e9
    return {"fwd_lse_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
            "bwd_ms_pct": {"p10": round(float(np.percentile(bt, 10)), 4), "p90": round(float(np.percentile(bt, 90)), 4),
                           "mean": round(float(bt.mean()), 4)},
            "bwd_over_fwd": round(b_ms / f_ms, 2),
            "train_tokens_per_s": round(W.batch * W.n / ((f_ms + b_ms) * 1e-3), 1),
            "bwd_useful_tflops": round(tflops, 2), "bwd_mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "bwd_algorithmic_bytes": bwd_bytes, "bwd_hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def fixed_blocks(P, W, q, k, v, steps=10, warmup=3):
    import numpy as np
    import torch
    block = np.maximum(1, np.rint(2.0 * np.asarray(W.sigmas, dtype=np.float64))).astype(np.int32)
    o = torch.empty_like(q)
    ws = torch.empty(P.workspace_bytes(W.heads_q, 1, W.n), dtype=torch.uint8, device=q.device)
    for _ in range(warmup):
        P.fixed_blocks(q, k, v, block, causal=W.causal, out=o, workspace=ws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        P.fixed_blocks(q, k, v, block, causal=W.causal, out=o, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps, block


def crossover(P, synth, dev, ns, steps=5):
    import torch
    out = {"n": [], "plsh_ms": [], "dense_ms": []}
    for n in ns:
        W = synth.Workload(f"mistral-n{n}", 1, 32, 8, n, 128, "bf16", synth.alibi_sigmas(32), 20, True, 0, 1003)
        q, k, v = synth.qkv_torch(1, 32, 8, n, 128, "bf16", 1003, dev)
        run = Runner(P, W, q, k, v, torch.empty_like(q), dev)
        wall = time_steps(run, steps, 2)
        dms = dense_alibi(P, W, q, k, v, steps=steps, warmup=2)
        out["n"].append(n)
        out["plsh_ms"].append(round(1e3 * wall / steps, 4))
        out["dense_ms"].append(round(dms, 4))
        del q, k, v, run
        torch.cuda.empty_cache()
    cross = None
    for n, a, b in zip(out["n"], out["plsh_ms"], out["dense_ms"]):
        if a < b:
            cross = n
            break
    out["crossover_n"] = cross
    return out


def long_point(P, synth, dev, dense_ms, steps=5):
    """The long-context workload (n = 131072, s = 32, causal, Mistral head
    layout) as one step of the whole path, against dense exact ALiBi at the
    same n (the dense kernel does not depend on s)."""
    import numpy as np
    import torch
    W = synth.WORKLOADS["long"]
    q, k, v = synth.qkv_torch(W.batch, W.heads_q, W.heads_kv, W.n, W.head_dim, W.dtype, W.data_seed, dev)
    run = Runner(P, W, q, k, v, torch.empty_like(q), dev)
    wall = time_steps(run, steps, 2)
    ms = 1e3 * wall / steps
    kms = float(np.median(kernel_times(run, 5, cold=True)))
    abytes = algorithmic_bytes(W) + bin_buffer_bytes(W, P, run.ws)
    del q, k, v, run
    torch.cuda.empty_cache()
    out = {"workload": "long-context", "n": W.n, "s": W.s, "plsh_ms": round(ms, 4),
           "kernel_ms_cold_cache": round(kms, 4), "tokens_per_s": round(W.batch * W.n / (ms * 1e-3), 1),
           "hbm_frac_cold_cache": round(abytes / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if dense_ms is not None:
        out["dense_ms"] = round(dense_ms, 4)
        out["speedup_plsh_vs_dense"] = round(dense_ms / ms, 2)
    return out


def workload_point(P, synth, dev, name, steps=20):
    """One workload as a step of the whole path: tokens/s of the step, the
    attention kernel's median with caches evicted and back to back, and the
    cold-cache HBM fraction."""
    import numpy as np
    import torch
    W = synth.WORKLOADS[name]
    q, k, v = synth.qkv_torch(W.batch, W.heads_q, W.heads_kv, W.n, W.head_dim, W.dtype, W.data_seed, dev)
    run = Runner(P, W, q, k, v, torch.empty_like(q), dev)
    wall = time_steps(run, steps, 5)
    ms = 1e3 * wall / steps
    cold = float(np.median(kernel_times(run, 10, cold=True)))
    warm = float(np.median(kernel_times(run, 10, cold=False)))
    abytes = algorithmic_bytes(W) + bin_buffer_bytes(W, P, run.ws)
    del q, k, v, run
    torch.cuda.empty_cache()
    return {"batch": W.batch, "heads_q": W.heads_q, "heads_kv": W.heads_kv, "n": W.n, "head_dim": W.head_dim,
            "dtype": W.dtype, "s": W.s, "causal": W.causal, "step_ms": round(ms, 5),
            "tokens_per_s": round(W.batch * W.n / (ms * 1e-3), 1), "kernel_ms_cold_cache": round(cold, 5),
            "kernel_ms_warm": round(warm, 5),
            "hbm_frac_cold_cache": round(abytes / (cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def convergence(P, dev, n=131072, sigma=256.0, ss=(2, 4, 8, 16, 32, 64, 128), seeds=3, max_steps=400):
    """Both error norms of the mask mean against L* over s, one head."""
    import numpy as np
    import torch
    import synth
    out = {"n": n, "sigma": sigma, "s": list(ss), "seeds": seeds, "spectral": [], "maxnorm": [], "ms": [],
           "lanczos_steps": [], "lanczos_converged": []}
    ws = torch.empty(P.error_workspace_bytes(n, max(ss), max_steps), dtype=torch.uint8, device=dev)
    for s in ss:
        sp, mx, ms, st = [], [], [], []
        for seed in range(seeds):
            delta, u = P.draw_hashes(1000 + seed, [sigma], s)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            r = P.error_norms(sigma, delta[0], u[0], n, max_steps=max_steps, tol=1e-9, seed=seed, workspace=ws)
            ms.append(1e3 * (time.perf_counter() - t0))
            sp.append(r["spectral"])
            mx.append(r["maxnorm"])
            st.append(r["steps"])
        out["spectral"].append(float(np.mean(sp)))
        out["maxnorm"].append(float(np.mean(mx)))
        out["ms"].append(round(float(np.mean(ms)), 2))
        out["lanczos_steps"].append(int(np.max(st)))
        out["lanczos_converged"].append(bool(np.max(st) < max_steps))
    # log-log slopes over s >= 8, past the small-s regime where the max norm sits near 1
    sel = np.asarray(ss) >= 8
    ls = np.log(np.asarray(ss, dtype=np.float64))[sel]
    out["slope_spectral"] = round(float(np.polyfit(ls, np.log(np.asarray(out["spectral"])[sel]), 1)[0]), 3)
    out["slope_maxnorm"] = round(float(np.polyfit(ls, np.log(np.asarray(out["maxnorm"])[sel]), 1)[0]), 3)
    out["spectral"] = [round(x, 6) for x in out["spectral"]]
    out["maxnorm"] = [round(x, 6) for x in out["maxnorm"]]
    return out


def copy_calibration(dev, nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling HBM counters."""
    import torch
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).normal_()
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {nbytes} bytes = {reps * nbytes} bytes read and written")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="mistral")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-crossover", action="store_true")
    ap.add_argument("--no-convergence", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-literal", action="store_true")
    ap.add_argument("--no-workloads", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true", help="only run a 1 GiB device copy (counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): the Positional-LSH path here "
            "is single-GPU; multi-GPU sharding is a design note, not built.")
        sys.exit(2)

    import numpy as np
    import torch

    import randomized_positional_lsh_amd as P
    import synth

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(dev)
        return

    W = synth.WORKLOADS[args.workload]
    log(f"workload {W.name}: B={W.batch} Hq={W.heads_q} Hkv={W.heads_kv} n={W.n} d={W.head_dim} {W.dtype} "
        f"s={W.s} causal={W.causal}")
    q, k, v = synth.qkv_torch(W.batch, W.heads_q, W.heads_kv, W.n, W.head_dim, W.dtype, W.data_seed, dev)
    o = torch.empty_like(q)
    run = Runner(P, W, q, k, v, o, dev)
    # the separate passes first (the per-step distribution, the kernel with
    # and without cache eviction): they run on the same buffers, so the timed
    # loop that follows starts on a GPU at its steady clocks with the
    # buffers' pages mapped, whatever its own warmup count
    for _ in range(50):  # the device's clocks ramp up under the first milliseconds of load
        run.step()
    steps_ms = step_times(run, 20)
    warm = kernel_times(run, 50, cold=False)
    cold = kernel_times(run, 50, cold=True)
    wall = time_steps(run, args.steps, args.warmup)
    ms_step = 1e3 * wall / args.steps
    tokens = W.batch * W.n
    # the two-launch form of the same step, for reference; it also leaves the
    # host copy of this draw in run.delta / run.u for the legs below
    for _ in range(20):
        run.two_launch()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(100):
        run.two_launch()
    torch.cuda.synchronize()
    ms_two = 1e3 * (time.perf_counter() - t0) / 100
    value = tokens / (wall / args.steps)
    log(f"step {ms_step:.4f} ms ({args.steps} timed steps after {args.warmup} warmup steps)")
    kern_ms = float(np.median(cold))
    warm_ms = float(np.median(warm))
    log(f"step median {np.median(steps_ms):.4f} ms; kernel median {kern_ms:.4f} ms with caches evicted, "
        f"{warm_ms:.4f} ms back to back; two-launch step {ms_two:.4f} ms")

    delta = run.delta.reshape(W.heads_q, W.s).copy()
    u = run.u.reshape(W.heads_q, W.s).copy()
    bbytes = bin_buffer_bytes(W, P, run.ws)
    abytes = algorithmic_bytes(W) + bbytes
    achieved = abytes / (kern_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_sha") == kernel_sha() and tr.get("workload") == W.name:
            traffic = int(tr["bytes_per_launch"])
    flops = useful_flops(W, P, run.ws)
    tflops = flops / (kern_ms * 1e-3) / 1e12
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "plpsh fwd_kernel (bins of each query tile + attention)",
                "cache": "L2 and last-level cache evicted before each launch",
                "kernel_ms": round(kern_ms, 5), "kernel_ms_pct": pct(cold), "algorithmic_bytes": abytes,
                "bin_buffer_bytes": bbytes,
                "useful_tflops": round(tflops, 2), "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "kernel_ms_warm": round(warm_ms, 5), "kernel_ms_warm_pct": pct(warm),
                "frac_warm": round(abytes / (warm_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "outside_kernel_ms": round(ms_step - warm_ms, 5)}

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": W.dtype, "data": "synthetic N(0,1) Q/K/V, hash seed 0",
        "config": {"workload": f"{W.name}-layer", "batch": W.batch, "heads_q": W.heads_q, "heads_kv": W.heads_kv,
                   "n": W.n, "head_dim": W.head_dim, "s": W.s, "causal": W.causal,
                   "sigma": "2^(8(h+1)/H)", "parallelism": "single GPU"},
        "step_ms": pct(steps_ms),
        "two_launch": {"step_ms": round(ms_two, 5), "tokens_per_s": round(tokens / (ms_two * 1e-3), 1)},
        "roofline": roofline,
    }
    if W.dtype == "bf16" and not args.no_backward:
        line["backward"] = backward(P, W, run, flops)
        log(f"backward {line['backward']}")
    if not args.no_literal:
        lms = literal(run)
        line["literal"] = {"kernel_ms": round(lms, 4), "fused_kernel_ms": round(warm_ms, 4),
                           "slowdown_vs_fused": round(lms / warm_ms, 2)}
        log(f"literal per-hash attention kernel {lms:.4f} ms")
    if not args.no_dense:
        dms = dense_alibi(P, W, q, k, v)
        line["dense_alibi"] = {"ms": round(dms, 4), "tokens_per_s": round(tokens / (dms * 1e-3), 1),
                               "speedup_plsh_vs_dense": round(dms / ms_step, 2)}
        log(f"dense exact ALiBi {dms:.4f} ms")
        fms, block = fixed_blocks(P, W, q, k, v)
        line["fixed_blocks"] = {"ms": round(fms, 4), "tokens_per_s": round(tokens / (fms * 1e-3), 1),
                                "block": "round(2 sigma_h)", "block_min": int(block.min()),
                                "block_max": int(block.max())}
        log(f"fixed blocks {fms:.4f} ms")
    if not args.no_workloads:
        line["workloads"] = {}
        for name in ("tiny", "small", "qwen3", "long"):
            if name != W.name:
                line["workloads"][name] = workload_point(P, synth, dev, name)
                log(f"workload {name} {line['workloads'][name]}")
    if not args.no_crossover and W.name == "mistral":
        del o
        line["crossover"] = crossover(P, synth, dev, [512, 1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072])
        log(f"crossover {line['crossover']}")
        cx = line["crossover"]
        line["long_context"] = long_point(P, synth, dev, cx["dense_ms"][-1] if cx["n"][-1] == 131072 else None)
        log(f"long context {line['long_context']}")
    if not args.no_convergence:
        line["convergence"] = convergence(P, dev)
        log(f"convergence {line['convergence']}")
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(W, q, k, v, delta, u, args.cpu_seconds)
        log(f"cpu baseline {line['cpu_baseline']}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
