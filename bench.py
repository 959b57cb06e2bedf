#!/usr/bin/env python3
"""Benchmark of the KLA operator on one MI355X.

One step = one chunkwise-prefill call (kla_chunk_fwd) over the prefill
workload B=4, H=16, T=4096, dk=dv=128, chunk 64, bf16 inputs, fp32 state:
every prefill step of the operator (fused loader with ||k||^2 and beta, Gram
and decay mask, blocked triangular solve, T applied to the chunk, sequential
state scan, causal output, final states) runs inside that call.  Inputs are
seeded synthetic tensors resident in HBM before timing starts.

Also measured in the same run and reported in the same JSON line:
  * decode: 512 consecutive kla_decode_step calls, N=256 sequences x H=16,
    128x128 fp32 state (HBM-bound; reported as GB/s);
  * backward: kla_chunk_bwd on the prefill workload (steps/10 timed calls);
  * the other prefill workloads (T=65536 dv=256; 32 packed sequences, H=32);
  * gdn: the same kernels with the update coefficient given;
  * pgdn: the preconditioned variant, prefill (general kernel) and decode;
  * cpu_baseline: the fp64 CPU oracle on this host's cores (a process pool),
    on the whole prefill workload and bounded samples of the others.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--mode all|prefill|decode|backward|prefill-other|pgdn]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KLA prefill tokens/s + TFLOP/s (H=16,d=128) and decode GB/s, 1×MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published (no sparsity)


def prefill_algorithmic(B, H, T, dk, dv, C, n_states_read, n_states_written, N):
    """Fixed-formula work of one prefill call (independent of the implementation).

    flops per token-head: 2C(3dk + 2dv) + 6 dk dv  (dense chunk form: K K^T,
      Q K^T, T applied to the chunk, K S, Q S, P U~, K^T U~)
    bytes per token-head: q, k, v, g, eta read and o written once (bf16),
      plus 4 dk dv per state read or written (N sequences x H heads).
    """
    th = B * H * T
    flops = th * (2 * C * (3 * dk + 2 * dv) + 6 * dk * dv)
    byts = th * (2 * (2 * dk + dv) + 2 * 2 + 2 * dv) + 4 * dk * dv * N * H * (n_states_read + n_states_written)
    return flops, byts


def backward_algorithmic(B, H, T, dk, dv, C, n_states_read, n_states_written, N):
    """Fixed-formula work of one backward call (independent of the implementation).

    flops per token-head: 12 dk dv + 8 C dv + 6 C dk + 4 C^2, the dense products of the
      chunk form's reverse mode counted once each (dU, dX, dS, dP, dW, dA, dQ, dK); the
      forward quantities a backward recomputes are not counted.
    bytes per token-head: q, k, v, do, g, eta read and dq, dk, dv written once (bf16),
      dg, deta written (fp32), plus 4 dk dv per state read or written per (sequence, head).
    """
    th = B * H * T
    flops = th * (12 * dk * dv + 8 * C * dv + 6 * C * dk + 4 * C * C)
    byts = (th * (2 * (2 * dk + 2 * dv) + 2 * 2 + 2 * (2 * dk + dv) + 2 * 4)
            + 4 * dk * dv * N * H * (n_states_read + n_states_written))
    return flops, byts


def decode_algorithmic(N, H, dk, dv):
    """Bytes of one decode step: state read + written (fp32), q/k/v/g/eta read, o written (bf16)."""
    per_head = 8 * dk * dv + 2 * (2 * dk + dv) + 2 * 2 + 2 * dv
    return N * H * per_head, N * H * 6 * dk * dv


def recorded_traffic(profile_md, *kernel_srcs):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when a kernel source has changed since those counters were taken (the
    summary records the sha256 of the listed sources' bytes, concatenated in
    order)."""
    import hashlib
    try:
        txt = open(os.path.join(ROOT, "profiles", profile_md)).read()
        src = b"".join(open(os.path.join(ROOT, f), "rb").read() for f in kernel_srcs)
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in txt.splitlines() if ": " in line and line[:1].isalpha())
    if fields.get("kernel_source_sha256", "").strip() != hashlib.sha256(src).hexdigest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_launches(fn, steps, stream):
    """Mean duration (ms) of one call over `steps` back-to-back calls, from two
    HIP events recorded on the launch stream around all of them (no event
    between calls, so the GPU runs the calls as it would in a loop), and the
    host wall time of the same region."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for i in range(steps):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return a.elapsed_time(b) / steps, wall


def bench_prefill(steps, warmup):
    import torch
    from gated_delta_rule_kla_amd import inputs, kla

    dev = torch.device("cuda:0")
    x = _workload(1)
    B, H, T, dk, dv = x.dims
    q, k, v, g, eta = (t.to(dev) for t in (x.q, x.k, x.v, x.g, x.eta))
    o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(kla.chunk_workspace_bytes(B, H, T, dk, dv, x.chunk, q.dtype), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(_i):
        kla.chunk_fwd(q, k, v, g, eta, x.eps, None, None, chunk=x.chunk, out=o, final_state=S, workspace=ws)

    for i in range(warmup):
        step(i)
    ms, wall = time_launches(step, steps, stream)
    flops, byts = prefill_algorithmic(B, H, T, dk, dv, x.chunk, 0, 1, B)
    return dict(ms=ms, wall_ms=wall * 1e3 / steps, tokens=B * T, flops=flops, bytes=byts,
                dims=(B, H, T, dk, dv, x.chunk))


def bench_prefill_other(steps, warmup, only=None):
    """The other two prefill workloads, each timed as one kla_chunk_fwd call per
    step: the long-context one (B=1 H=16 T=65536 dk=128 dv=256, no initial state)
    and the 32 packed sequences of log-uniform lengths (H=32, cu_seqlens, nonzero
    initial states).  Reported beside the main line, not as the metric.  The
    workspace is kla_chunk_workspace_bytes', so kla_chunk_fwd takes its own choice
    of segments ("segmented": the long-context workload runs the segment-parallel
    scan, the packed batch does not)."""
    import torch
    from gated_delta_rule_kla_amd import inputs, kla

    dev = torch.device("cuda:0")
    res = {}
    for i in ((2, 4) if only is None else (only,)):
        x = _workload(i)
        B, H, T, dk, dv = x.dims
        q, k, v, g, eta = (t.to(dev) for t in (x.q, x.k, x.v, x.g, x.eta))
        s0 = x.initial_state.to(dev) if x.initial_state is not None else None
        cu = x.cu_seqlens.to(dev) if x.cu_seqlens is not None else None
        cu_h = x.cu_seqlens if x.cu_seqlens is not None else None
        N = (x.cu_seqlens.numel() - 1) if x.cu_seqlens is not None else B
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
        S = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
        ws_bytes = kla.chunk_workspace_bytes(B, H, T, dk, dv, x.chunk, q.dtype, cu_seqlens_host=cu_h)
        segmented = ws_bytes > kla.chunk_workspace_bytes(B, H, T, dk, dv, x.chunk, q.dtype, cu_seqlens_host=cu_h,
                                                         seg_chunks=0)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        stream = torch.cuda.current_stream(dev)

        def step(_i):
            kla.chunk_fwd(q, k, v, g, eta, x.eps, s0, cu, chunk=x.chunk, cu_seqlens_host=cu_h,
                          out=o, final_state=S, workspace=ws)

        for j in range(warmup):
            step(j)
        ms, _ = time_launches(step, steps, stream)
        flops, byts = prefill_algorithmic(B, H, T, dk, dv, x.chunk, 1 if s0 is not None else 0, 1, N)
        sec = ms * 1e-3
        res[inputs.CONFIGS[i]] = {
            "ms_per_call": ms, "segmented": bool(segmented), "tokens/s": B * T / sec, "tflops": flops / sec / 1e12,
            "GB/s": byts / sec / 1e9, "hbm_frac": byts / sec / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes_per_launch": byts, "algorithmic_flops_per_launch": flops}
        del q, k, v, g, eta, o, S, ws, s0, cu
        torch.cuda.empty_cache()
    return res


def bench_backward(steps, warmup):
    """kla_chunk_bwd on the prefill workload: upstream gradients dL/do (bf16) and
    dL/dS_final (fp32) seeded, the initial-state gradient requested."""
    import torch
    from gated_delta_rule_kla_amd import inputs, kla

    dev = torch.device("cuda:0")
    x = _workload(1)
    B, H, T, dk, dv = x.dims
    q, k, v, g, eta = (t.to(dev) for t in (x.q, x.k, x.v, x.g, x.eta))
    do_h, ds_h = inputs.make_upstream(x, 101)
    do, ds = do_h.to(dev), ds_h.to(dev)
    ws = torch.empty(kla.chunk_bwd_workspace_bytes(B, H, T, dk, dv, x.chunk, q.dtype), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(_i):
        kla.chunk_bwd(q, k, v, g, eta, do, x.eps, None, ds, None, chunk=x.chunk, workspace=ws)

    for i in range(warmup):
        step(i)
    ms, wall = time_launches(step, steps, stream)
    flops, byts = backward_algorithmic(B, H, T, dk, dv, x.chunk, 1, 1, B)
    return dict(ms=ms, wall_ms=wall * 1e3 / steps, tokens=B * T, flops=flops, bytes=byts,
                ws_bytes=ws.numel(), dims=(B, H, T, dk, dv, x.chunk))


def bench_gdn(steps, warmup, decode_steps=512):
    """The same kernels in gated-delta-rule mode (kla_gdn_*: the update
    coefficient given instead of the Kaczmarz step), on the prefill and decode
    workloads with unit-length keys: the operator-level form of the pages'
    KLA-versus-GDN latency comparison."""
    import torch
    from gated_delta_rule_kla_amd import inputs, kla

    dev = torch.device("cuda:0")
    x = inputs.unit_keys(_workload(1))
    B, H, T, dk, dv = x.dims
    q, k, v, g, beta = (t.to(dev) for t in (x.q, x.k, x.v, x.g, x.eta))
    o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(kla.chunk_workspace_bytes(B, H, T, dk, dv, x.chunk, q.dtype), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def pstep(_i):
        kla.gdn_chunk_fwd(q, k, v, g, beta, None, None, chunk=x.chunk, out=o, final_state=S, workspace=ws)

    for i in range(warmup):
        pstep(i)
    p_ms, _ = time_launches(pstep, steps, stream)
    del q, k, v, g, beta, o, S, ws
    d = inputs.unit_keys(_workload(3) if decode_steps == 512 else inputs.decode_config(steps=decode_steps))
    dq, dk_, dv_, dg, db = (t.to(dev) for t in (d.q, d.k, d.v, d.g, d.eta))
    st = d.state.to(dev)
    do = torch.empty((d.q.shape[1], d.q.shape[2], d.v.shape[-1]), dtype=dq.dtype, device=dev)

    def dstep(i):
        kla.gdn_decode_step(dq[i], dk_[i], dv_[i], dg[i], db[i], st, out=do)

    for i in range(64):
        dstep(i % decode_steps)
    d_ms, _ = time_launches(dstep, decode_steps, stream)
    return dict(prefill_ms=p_ms, decode_ms=d_ms, tokens=B * T)


def bench_pgdn(steps, warmup, decode_steps=64):
    """PGDN (kla_pgdn_chunk_fwd / kla_pgdn_decode_step: the preconditioned gated
    delta rule, coefficient given, band 1.5) on the prefill workload and the first
    steps of the decode workload, both with unit-length keys: the pipelined prep
    and scan kernels after the key-accumulator and write-key passes, and the
    HBM-tuned decode kernel."""
    import torch
    from gated_delta_rule_kla_amd import inputs, kla

    dev = torch.device("cuda:0")
    x = inputs.unit_keys(_workload(1))
    B, H, T, dk, dv = x.dims
    q, k, v, g, beta = (t.to(dev) for t in (x.q, x.k, x.v, x.g, x.eta))
    o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    A = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, kla.pgdn_chunk_workspace_bytes(B, H, T, dk, dv, x.chunk, q.dtype)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def pstep(_i):
        kla.pgdn_chunk_fwd(q, k, v, g, beta, x.eps, "given", 1.5, None, None, chunk=x.chunk, out=o,
                           final_state=S, final_acc=A, workspace=ws)

    for i in range(warmup):
        pstep(i)
    p_ms, _ = time_launches(pstep, steps, stream)
    _, p_bytes = prefill_algorithmic(B, H, T, dk, dv, x.chunk, 0, 1, B)
    p_bytes += 4 * dk * B * H  # the final accumulator
    del q, k, v, g, beta, o, S, A, ws
    d = inputs.unit_keys(_workload(3))
    N, Hd, dkd = d.q.shape[1:]
    dvd = d.v.shape[-1]
    dq, dk_, dv_, dg, db = (t[:decode_steps].to(dev) for t in (d.q, d.k, d.v, d.g, d.eta))
    st = d.state.to(dev)
    acc = torch.zeros((N, Hd, dkd), dtype=torch.float32, device=dev)
    do = torch.empty((N, Hd, dvd), dtype=dq.dtype, device=dev)

    def dstep(i):
        kla.pgdn_decode_step(dq[i], dk_[i], dv_[i], dg[i], db[i], d.eps, st, acc, "given", 1.5, out=do)

    for i in range(16):
        dstep(i % decode_steps)
    d_ms, _ = time_launches(dstep, decode_steps, stream)
    d_bytes, _ = decode_algorithmic(N, Hd, dkd, dvd)
    d_bytes += 8 * dkd * N * Hd  # the accumulator read and written
    del st, acc
    torch.cuda.empty_cache()
    return {"workload": f"PGDN (given coefficient, band 1.5, unit-length keys): prefill B={B} H={H} T={T} "
                        f"dk={dk} dv={dv} chunk={x.chunk} bf16; decode "
                        f"N={N} H={Hd} dk={dkd} dv={dvd}, {decode_steps} consecutive steps",
            "prefill_ms_per_call": p_ms, "prefill_tokens/s": B * T / (p_ms * 1e-3),
            "prefill_GB/s": p_bytes / p_ms / 1e6, "prefill_hbm_frac": p_bytes / p_ms / 1e6 / HBM_PEAK_GBS,
            "decode_ms_per_step": d_ms, "decode_GB/s": d_bytes / d_ms / 1e6,
            "decode_hbm_frac": d_bytes / d_ms / 1e6 / HBM_PEAK_GBS}


def bench_decode_large(steps_total=64, warmup=16, N=1024):
    """The decode step with a state four times the 256 MB Infinity Cache (N=1024
    sequences x 16 heads x 128 x 128 fp32 = 1 GiB), so that no step can find
    the previous step's writes in that cache: the figure checks that the decode
    rate is HBM's, not the cache's."""
    import torch
    from gated_delta_rule_kla_amd import inputs, kla

    dev = torch.device("cuda:0")
    d = inputs.decode_config(steps=steps_total, N=N)
    H, dk = d.q.shape[2:]
    dv = d.v.shape[-1]
    q, k, v, g, eta = (t.to(dev) for t in (d.q, d.k, d.v, d.g, d.eta))
    st = d.state.to(dev)
    o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        kla.decode_step(q[i], k[i], v[i], g[i], eta[i], d.eps, st, out=o)

    for i in range(warmup):
        step(i % steps_total)
    ms, _ = time_launches(step, steps_total, stream)
    byts, _ = decode_algorithmic(N, H, dk, dv)
    del q, k, v, g, eta, st, o
    torch.cuda.empty_cache()
    return {"workload": f"KLA decode step, N={N} H={H} dk={dk} dv={dv}, fp32 state of {N * H * dk * dv * 4 >> 20} "
                        f"MiB, {steps_total} consecutive steps",
            "ms_per_step": ms, "GB/s": byts / ms / 1e6, "hbm_frac": byts / ms / 1e6 / HBM_PEAK_GBS}


def bench_decode(steps_total=512, warmup=64):
    import torch
    from gated_delta_rule_kla_amd import inputs, kla

    dev = torch.device("cuda:0")
    d = _workload(3) if steps_total == 512 else inputs.decode_config(steps=steps_total)
    N, H, dk = d.q.shape[1:]
    dv = d.v.shape[-1]
    q, k, v, g, eta = (t.to(dev) for t in (d.q, d.k, d.v, d.g, d.eta))
    st = d.state.to(dev)
    o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        kla.decode_step(q[i], k[i], v[i], g[i], eta[i], d.eps, st, out=o)

    for i in range(warmup):
        step(i % steps_total)
    ms, wall = time_launches(step, steps_total, stream)
    byts, flops = decode_algorithmic(N, H, dk, dv)
    return dict(ms=ms, wall_ms=wall * 1e3 / steps_total, bytes=byts, flops=flops, N=N, H=H, dk=dk, dv=dv,
                steps=steps_total)


# Generated workloads, kept for the whole run: the CPU baseline and the GPU legs
# use the same seeded tensors (generating the largest takes tens of seconds).
# The CPU-baseline pool's workers are forked after it is filled, so they inherit
# it without copying (they only read it).
_CPU_WORK = {}


def _workload(i):
    from gated_delta_rule_kla_amd import inputs
    if i not in _CPU_WORK:
        _CPU_WORK[i] = inputs.decode_config() if i == 3 else inputs.prefill_config(i)
    return _CPU_WORK[i]


def _cpu_task(task):
    """One (workload, sequence, head) unit of the oracle, timed in a worker."""
    import numpy as np
    from gated_delta_rule_kla_amd import inputs
    from oracle import kla_decode_step, kla_recurrence

    f = inputs.to_f64
    kind, i, a, b, h = task
    t0 = time.perf_counter()
    if kind == "prefill":
        x = _CPU_WORK[i]
        if x.cu_seqlens is None:
            row, lo, hi, n = a, 0, x.q.shape[2], a
        else:
            row, lo, hi, n = 0, int(x.cu_seqlens[a]), int(x.cu_seqlens[a + 1]), a
        s0 = None if x.initial_state is None else f(x.initial_state[n, h])
        kla_recurrence(f(x.q[row, h, lo:hi]), f(x.k[row, h, lo:hi]), f(x.v[row, h, lo:hi]),
                       f(x.g[row, h, lo:hi]), f(x.eta[row, h, lo:hi]), x.eps, s0)
        units = hi - lo
    else:  # decode: every step of one (sequence, head)
        d = _CPU_WORK[i]
        S = f(d.state[a:a + 1, h:h + 1])
        for s in range(d.q.shape[0]):
            _, S = kla_decode_step(f(d.q[s, a:a + 1, h:h + 1]), f(d.k[s, a:a + 1, h:h + 1]),
                                   f(d.v[s, a:a + 1, h:h + 1]), f(d.g[s, a:a + 1, h:h + 1]),
                                   f(d.eta[s, a:a + 1, h:h + 1]), d.eps, S)
        units = d.q.shape[0]
    return units, time.perf_counter() - t0


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    import torch
    torch.set_num_threads(1)
    threadpool_limits(1)


def cpu_baseline():
    """The fp64 oracle, as it stands, on this host's cores: a process pool over
    (sequence, head) pairs, one BLAS thread per worker.  Runs before anything
    touches the GPU (the workers are forked from this process).

    Samples (each pair runs in full, every token or step):
      0  the tiny fp32 workload, whole;
      1  the B=4 H=16 T=4096 prefill workload, whole (64 pairs) -- `value`;
      2  the T=65536 dv=256 workload, heads 0, 5, 10, 15 (4 of 16 pairs);
      3  the decode workload, 64 of 4096 (sequence, head) pairs over all 512 steps;
      4  the 32 packed sequences, heads 0, 4, ..., 28 (256 of 1024 pairs).
    Tokens/s for a sample = tokens of the pairs it ran (one head each) / wall
    seconds x heads of the workload, i.e. the workload's own token rate if the
    oracle kept that speed on every head."""
    import multiprocessing as mp

    from gated_delta_rule_kla_amd import inputs

    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    for i in range(5):
        _workload(i)
    plans = {
        0: [("prefill", 0, 0, 0, 0)],
        1: [("prefill", 1, b, 0, h) for b in range(4) for h in range(16)],
        2: [("prefill", 2, 0, 0, h) for h in (0, 5, 10, 15)],
        3: [("decode", 3, n, 0, h) for n, h in zip(range(0, 256, 4), [i % 16 for i in range(64)])],
        4: [("prefill", 4, n, 0, h) for n in range(32) for h in range(0, 32, 4)],
    }
    heads = {0: 1, 1: 16, 2: 16, 3: 16, 4: 32}
    per = {}
    ctx = mp.get_context("fork")
    with ctx.Pool(cores, initializer=_cpu_worker_init) as pool:
        for i, tasks in plans.items():
            t0 = time.perf_counter()
            res = pool.map(_cpu_task, tasks, chunksize=1)
            wall = time.perf_counter() - t0
            units = sum(u for u, _ in res)
            busy = sum(t for _, t in res)
            if i == 3:
                per[inputs.CONFIGS[i]] = {
                    "seconds": wall, "pairs": len(tasks), "steps": units // len(tasks),
                    "head_steps/s": units / wall, "tokens/s": units / wall / heads[i],
                    "worker_seconds": busy}
            else:
                per[inputs.CONFIGS[i]] = {
                    "seconds": wall, "pairs": len(tasks), "token_heads": units,
                    "tokens/s": units / wall / heads[i], "worker_seconds": busy}
    head = per[inputs.CONFIGS[1]]
    return dict(value=head["tokens/s"], unit="tokens/s", cores=cores, kind="oracle",
                sample=(f"fp64 numpy token recurrence over all 64 (sequence, head) pairs of the B=4 H=16 "
                        f"T=4096 dk=dv=128 workload, a process pool of {cores} workers with one BLAS "
                        f"thread each, {head['seconds']:.1f} s wall; the other workloads on the "
                        f"samples listed in per_workload"),
                per_workload=per)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--mode", choices=["all", "prefill", "decode", "backward", "prefill-other", "pgdn"],
                    default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", type=int, choices=[2, 4],
                    help="prefill-other: time only this workload (2: T=65536 dv=256, 4: 32 packed sequences)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (for HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this operator build measures one GPU only (no multi-GPU path); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    # the CPU baseline forks its worker pool, so it runs before anything touches the GPU
    cpu = None
    if args.mode == "all" and not args.no_cpu_baseline:
        cpu = cpu_baseline()

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) q/k/v, key scale exp(N(0,0.5)), g=-softplus(N(0,1)), "
                   "eta=sigmoid(N(0,1)))"}

    if args.copy_calibration:
        a = torch.empty(64 << 20, dtype=torch.float32, device="cuda:0").fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = {"read": a.numel() * 4, "written": b.numel() * 4}

    if args.mode in ("all", "prefill"):
        p = bench_prefill(args.steps, args.warmup)
        B, H, T, dk, dv, C = p["dims"]
        sec = p["ms"] * 1e-3
        gbs = p["bytes"] / sec / 1e9
        tfl = p["flops"] / sec / 1e12
        out.update({
            "value": p["tokens"] / sec, "unit": "tokens/s", "ms_per_step": p["ms"],
            "wall_ms_per_step": p["wall_ms"],
            "config": {"workload": f"KLA chunkwise prefill, B={B} H={H} T={T} dk={dk} dv={dv} "
                                   f"chunk={C}, bf16 q/k/v/g/eta, fp32 state, no initial state",
                       "global_batch": B, "seq_len": T, "heads": H, "dk": dk, "dv": dv, "chunk": C},
            "tflops": tfl, "mfma_frac": tfl / BF16_PEAK_TFLOPS,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": recorded_traffic("kla_chunk_fwd_prefill_b4_h16_t4096_hbm.md",
                                                     "gated_delta_rule_kla_amd/csrc/kla_chunk.hip"),
                         "kernel": "kla_chunk_fwd: kla_chunk_prep_wave_kernel<128> then "
                                   "kla_chunk_kernel<bf16,64,128,2>, timed together per call",
                         "algorithmic_bytes_per_launch": p["bytes"],
                         "algorithmic_flops_per_launch": p["flops"],
                         "note": "arithmetic intensity 172.6 flop/B is below the bf16 ridge "
                                 "(312.5 flop/B), so HBM bounds this kernel; tflops/mfma_frac give "
                                 "the same launch against the bf16 MFMA peak"},
        })
    if args.mode in ("all", "decode"):
        d = bench_decode()
        sec = d["ms"] * 1e-3
        gbs = d["bytes"] / sec / 1e9
        dec = {"workload": f"KLA decode step, N={d['N']} H={d['H']} dk={d['dk']} dv={d['dv']}, fp32 state, "
                           f"{d['steps']} consecutive steps",
               "ms_per_step": d["ms"], "wall_ms_per_step": d["wall_ms"], "GB/s": gbs,
               "tokens/s": d["N"] / sec,
               "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": gbs / HBM_PEAK_GBS,
                            "traffic": recorded_traffic("kla_decode_kernel_n256_h16_hbm.md",
                                                        "gated_delta_rule_kla_amd/csrc/kla_decode.hip"),
                            "kernel": "kla_decode_kernel<bf16,128,128>",
                            "algorithmic_bytes_per_launch": d["bytes"]}}
        if args.mode == "decode":
            out.update({"value": gbs, "unit": "GB/s", "ms_per_step": d["ms"],
                        "config": {"workload": dec["workload"]}, "roofline": dec["roofline"]})
        if args.mode == "all":
            dec["beyond_infinity_cache"] = bench_decode_large()
        out["decode"] = dec
    if args.mode in ("all", "backward"):
        bw = bench_backward(max(1, args.steps // 10), max(1, args.warmup // 10))
        B, H, T, dk, dv, C = bw["dims"]
        sec = bw["ms"] * 1e-3
        gbs = bw["bytes"] / sec / 1e9
        bwd = {"workload": f"KLA chunkwise backward (kla_chunk_bwd), B={B} H={H} T={T} dk={dk} dv={dv} "
                           f"chunk={C}, bf16, upstream dL/do and dL/dS_final, dL/dS0 written",
               "ms_per_step": bw["ms"], "wall_ms_per_step": bw["wall_ms"], "tokens/s": bw["tokens"] / sec,
               "tflops": bw["flops"] / sec / 1e12, "workspace_bytes": bw["ws_bytes"],
               "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": gbs / HBM_PEAK_GBS,
                            "traffic": recorded_traffic("kla_chunk_bwd_b4_h16_t4096_hbm.md",
                                                        "gated_delta_rule_kla_amd/csrc/kla_chunk.hip",
                                                        "gated_delta_rule_kla_amd/csrc/kla_bwd.hip"),
                            "kernel": "kla_chunk_bwd: the forward prep (with the T image), the forward "
                                      "scan in states mode beside the adjoint scan, and the gradient "
                                      "kernel, timed together per call",
                            "algorithmic_bytes_per_launch": bw["bytes"],
                            "algorithmic_flops_per_launch": bw["flops"]}}
        if args.mode == "backward":
            out.update({"value": bw["tokens"] / sec, "unit": "tokens/s", "ms_per_step": bw["ms"],
                        "config": {"workload": bwd["workload"]}, "roofline": bwd["roofline"]})
        out["backward"] = bwd
    if args.mode == "prefill-other":
        out["prefill_other_workloads"] = bench_prefill_other(max(2, args.steps // 20), max(1, args.warmup // 10),
                                                             args.only)
    if args.mode in ("all", "pgdn"):
        out["pgdn"] = bench_pgdn(max(2, args.steps // 40), 1)
    if args.mode == "all":
        out["prefill_other_workloads"] = bench_prefill_other(max(2, args.steps // 20), max(1, args.warmup // 10))
        gd = bench_gdn(args.steps, args.warmup)
        gdn = {"workload": "the same prefill and decode workloads through kla_gdn_chunk_fwd / "
                           "kla_gdn_decode_step (update coefficient given; unit-length keys)",
               "prefill_ms_per_call": gd["prefill_ms"], "prefill_tokens/s": gd["tokens"] / (gd["prefill_ms"] * 1e-3),
               "decode_ms_per_step": gd["decode_ms"]}
        if "ms_per_step" in out:
            gdn["kla_over_gdn_prefill_time"] = out["ms_per_step"] / gd["prefill_ms"]
        if "decode" in out:
            gdn["kla_over_gdn_decode_time"] = out["decode"]["ms_per_step"] / gd["decode_ms"]
        out["gdn"] = gdn
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out))


if __name__ == "__main__":
    main()
