#!/usr/bin/env python3
"""Benchmark of routed exact-token attention (HGA) on one MI355X.

One step = one pass of the whole hot path over the Qwen3-30B-A3B-shaped
prefill layer (batch 1, 32 query / 4 KV heads, d=128, 32768 tokens, bf16,
C=64, g_s=16, F=2, L=8, K_c=16, K_g=32): hga_build_summaries (rotated key
cache + chunk / group summaries), hga_route (chunk and group top-K, visible
granule lists) and hga_attend (exact-token attention over those granules).
Inputs are resident in HBM before the timed region.

Also measured in the same run (extra fields of the one JSON line):
  decode  -- one decode step for 16 sequences x 65536 cached tokens
             (hga_decode_step, and hga_route + hga_attend, at position 65536,
             summaries precomputed), with the oracle on a few of its units;
  smalllm -- the SmallLM-shaped prefill (batch 4, 8/8 heads, d=64, 4096 tokens);
  tiny    -- the tiny f32 workload (1024 tokens, one head): us per step;
  cpu_baseline_small -- the oracle on the tiny and SmallLM workloads, on all
             BLAS threads and on one;
  host_tiered -- prefill over 131072 tokens with K/V in pinned host RAM
             (with and without the device cache of granules);
  decode_host_tier_stream -- the decode shape streamed token by token with
             its K/V history in pinned host RAM (DecodeSession);
  backward -- hga_attend_backward (dq, dk, dv) on the prefill's routes;
  cpu_baseline -- the CPU oracle on a bounded sample of the prefill step,
             and the GPU's routes and outputs checked on that sample.
Every timed region is preceded by half a second of dense matrix products, so
that the GPU runs at its steady clock whatever --warmup is.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       [--only prefill|decode|smalllm|tiny|host|stream|backward|copy|peaks]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "routed-attn prefill Mtok/s + decode us/step at 64K ctx; % of HBM/MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# warm tier of the host-tiered runs: a quarter of the 128K store's 32768
# granules (64 MiB of bf16 K+V)
WARM_TIER_SLOTS = 8192
ATTEND_PROFILE = os.path.join(ROOT, "profiles", "attend_mfma_qwen3_prefill_n32768.md")
ATTEND_SOURCES = ["attend.hip", "hga_device.h"]


def measured_peaks(torch):
    """The device's reachable peaks, measured with libhga_peak.so: dense bf16
    MFMA TFLOP/s (back-to-back 32x32x16 products, 8 workgroups per CU) and
    copy GB/s (read + write of 1 GiB; the better of a plain grid-stride copy
    kernel and torch's device copy)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "hierarchical_kv_routing_amd", "libhga_peak.so"))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    blocks, iters = cus * 8, 2000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")

    def mfma():
        assert lib.hga_peak_mfma(ctypes.c_void_p(sink.data_ptr()), blocks, iters, stream) == 0

    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").random_(0, 255)
    dst = torch.empty_like(src)

    def copy():
        assert lib.hga_peak_stream(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                   ctypes.c_int64(nbytes), cus * 8, stream) == 0

    def torch_copy():
        dst.copy_(src)

    out = {}
    for name, fn, work in (("mfma_bf16_tflops", mfma, blocks * 4 * 4 * iters * 32768 / 1e12),
                           ("hbm_copy_gbs", copy, 2 * nbytes / 1e9),
                           ("torch_copy_gbs", torch_copy, 2 * nbytes / 1e9)):
        for _ in range(30):  # tens of ms: the steady clock
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = work / (e0.elapsed_time(e1) / 10 * 1e-3)
    del src, dst, sink
    out["hbm_copy_gbs"] = max(out["hbm_copy_gbs"], out.pop("torch_copy_gbs"))  # the better copy
    return out


def recorded_traffic():
    """HBM bytes per attend launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (copy-calibrated), or None when the summary was taken
    on another version of the kernel source than the one built here."""
    import hashlib
    import re
    try:
        text = open(ATTEND_PROFILE).read()
    except OSError:
        return None
    t = re.search(r"attend traffic per launch: (\d+) bytes", text)
    h = re.search(r"kernel source sha256: ([0-9a-f]{64})", text)
    if t is None or h is None:
        return None
    cur = hashlib.sha256()
    for f in ATTEND_SOURCES:
        with open(os.path.join(ROOT, "hierarchical_kv_routing_amd", "csrc", f), "rb") as fh:
            cur.update(fh.read())
    return int(t.group(1)) if cur.hexdigest() == h.group(1) else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


CLOCK_WARMUP_S = 0.5


def warm_clock(torch, seconds=CLOCK_WARMUP_S):
    """Dense bf16 matrix products for ``seconds`` of wall time: the GPU leaves
    its idle clock (the first tens of ms of load otherwise run 10-20 %
    slower), so the timed steps see the steady clock whatever --warmup is."""
    a = torch.randn(8192, 8192, device="cuda:0", dtype=torch.bfloat16)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            b = a @ a
        torch.cuda.synchronize()
    del a, b


class Pipeline:
    """Device buffers and the three calls of one step."""

    def __init__(self, w, seed=0):
        import torch
        import hierarchical_kv_routing_amd as H
        self.H, self.torch, self.w = H, torch, w
        self.cfg = H.Config.from_workload(w)
        t0 = time.time()
        q, k, v = W.make_inputs(w, seed, threads=16)
        log(f"[bench] {w.name}: inputs generated in {time.time() - t0:.1f}s")
        dev = torch.device("cuda:0")
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.q = torch.from_numpy(q).to(dev).to(dt)
        self.k = torch.from_numpy(k).to(dev).to(dt)
        self.v = torch.from_numpy(v).to(dev).to(dt)
        self.q_np, self.k_np, self.v_np = q, k, v
        del q, k, v
        B, Hkv, cap, d = self.k.shape
        c = self.cfg
        self.k_rot = torch.empty_like(self.k)
        self.csum = torch.empty((B, Hkv, cap // c.chunk_size, d), dtype=torch.float32, device=dev)
        self.gsum = torch.empty((B, Hkv, cap // c.group_size, d), dtype=torch.float32, device=dev)
        self.ro = H.route_outputs(c, B, w.q_pos0, w.n_q, dev)
        self.out = torch.empty_like(self.q)
        aw = H.attend_workspace_bytes(c, B, w.q_pos0, w.n_q)
        self.aws = torch.empty(max(aw, 16), dtype=torch.uint8, device=dev)

    def build(self, lo=0, hi=None):
        self.H.build_summaries(self.cfg, self.k, lo, self.w.n_ctx if hi is None else hi,
                               self.k_rot, self.csum, self.gsum)

    def route(self):
        r = self.ro
        self.H.route(self.cfg, self.q, self.w.q_pos0, self.csum, self.gsum, self.k.shape[2],
                     r["chunk_idx"], r["group_idx"], r["granules"], r["granule_count"],
                     r["workspace"])

    def attend(self):
        r = self.ro
        self.H.attend(self.cfg, self.q, self.w.q_pos0, self.k_rot, self.v, r["granules"],
                      r["granule_count"], self.out, None, self.aws)


def timed_steps(torch, stages, steps, warmup):
    """Run ``warmup`` then ``steps`` steps of the stage list (after the clock
    warmup); events bracket the whole timed region and every stage (same
    stream as the launches)."""
    warm_clock(torch)
    for _ in range(warmup):
        for _, fn in stages:
            fn()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in stages] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(steps):
        for i, (_, fn) in enumerate(stages):
            ev[s][i][0].record()
            fn()
            ev[s][i][1].record()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    per_stage = {name: float(np.mean([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)]))
                 for i, (name, _) in enumerate(stages)}
    return total_ms / steps, per_stage


def visible_pairs(w, counts_np):
    """Sum over query rows (query, head) of the visible keys, from the
    granule counts (keys j <= i inside the current chunk are counted exactly)."""
    C, gs, G = w.chunk_size, w.group_size, w.group_ratio
    total = 0
    t0 = w.q_pos0 // C
    for u in range(counts_np.shape[2]):
        t = t0 + u
        qlo = max(t * C, w.q_pos0)
        qhi = min((t + 1) * C, w.q_pos0 + w.n_q)
        nq = qhi - qlo
        cnt = counts_np[:, :, u].astype(np.int64)
        # keys of the current chunk's granules come last in each list
        cur = (qhi - 1) // gs - (t * C) // gs + 1
        other = (cnt - cur) * gs
        causal = sum(i - t * C + 1 for i in range(qlo, qhi))
        total += int(G * (nq * other.sum() + causal * cnt.size))
    return total


def bench_prefill(args):
    import torch
    w = W.QWEN3_PREFILL
    pipe = Pipeline(w)
    ms, stage = timed_steps(torch, [("build_summaries", pipe.build), ("route", pipe.route),
                                    ("attend", pipe.attend)], args.steps, args.warmup)
    counts = pipe.ro["granule_count"].cpu().numpy()
    pairs = visible_pairs(w, counts)
    flops = 4.0 * w.head_dim * pairs              # QK^T and PV, 2 flops per MAC
    attend_tflops = flops / (stage["attend"] * 1e-3) / 1e12
    res = dict(ms=ms, stage_ms=stage, pairs=pairs, attend_flops=flops,
               attend_tflops=attend_tflops, tokens=w.n_q)
    return pipe, res


def bench_backward(args, pipe=None, pairs=None):
    """hga_attend_backward on the Qwen3-shaped prefill (routes and forward
    outputs of one forward step held fixed, a random dO): dq, dk, dv."""
    import torch
    import hierarchical_kv_routing_amd as H
    w = W.QWEN3_PREFILL
    if pipe is None:
        pipe = Pipeline(w)
        pipe.build()
        pipe.route()
    lse = torch.empty(pipe.q.shape[:3], dtype=torch.float32, device="cuda:0")
    H.attend(pipe.cfg, pipe.q, w.q_pos0, pipe.k_rot, pipe.v, pipe.ro["granules"],
             pipe.ro["granule_count"], pipe.out, lse, pipe.aws)
    if pairs is None:
        pairs = visible_pairs(w, pipe.ro["granule_count"].cpu().numpy())
    g = torch.Generator(device="cuda:0")
    g.manual_seed(7)
    d_out = torch.randn(pipe.q.shape, generator=g, device="cuda:0").to(torch.bfloat16)
    dq = torch.empty(pipe.q.shape, dtype=torch.float32, device="cuda:0")
    dk = torch.empty(pipe.k.shape, dtype=torch.float32, device="cuda:0")
    dv = torch.empty(pipe.k.shape, dtype=torch.float32, device="cuda:0")
    ws = torch.empty(max(H.attend_backward_workspace_bytes(pipe.cfg, w.batch, w.q_pos0, w.n_q), 16),
                     dtype=torch.uint8, device="cuda:0")

    def bwd():
        H.attend_backward(pipe.cfg, pipe.q, w.q_pos0, pipe.k_rot, pipe.v, pipe.ro["granules"],
                          pipe.ro["granule_count"], pipe.out, lse, d_out, dq, dk, dv, ws)
    ms, _ = timed_steps(torch, [("backward", bwd)], max(4, args.steps // 5), max(2, args.warmup // 5))
    flops = 8.0 * w.head_dim * pairs  # dP, dQ, dK, dV: 2 flops per MAC, 4 products
    return dict(workload=w.name, ms=ms, algorithmic_flops=flops, tflops=flops / (ms * 1e-3) / 1e12,
                frac_of_peak=flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                timing="HIP events around hga_attend_backward (D and Q', transposes, lists, dq, dk/dv partials, reduce)")


def graph_step_ms(torch, fns, steps, warmup=3):
    """Average time of one replay of a HIP graph that holds the calls fns
    (captured on a side stream after a few eager warmup runs there; the clock
    warmed before the replays)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warmup):
            for fn in fns:
                fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in fns:
            fn()
    warm_clock(torch)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def decode_bytes(w, counts):
    """Algorithmic bytes of one decode step: scanned chunk summaries, the
    group summaries of the chosen chunks, gathered K and V of the visible
    tokens, q in and o out."""
    B, Hkv, d = w.batch, w.n_kv_heads, w.head_dim
    t = w.q_pos0 // w.chunk_size
    n_mid = t - w.n_sink_chunks - max(w.n_recent_chunks, 1)
    keys = (counts - 1) * w.group_size + 1  # the current chunk holds one token
    return (B * Hkv * n_mid * d * 4 + B * Hkv * w.top_chunks * (w.chunk_size // w.group_size) * d * 4
            + int(keys.sum()) * d * 2 * 2 + 2 * B * w.n_q_heads * d * 2)


def bench_decode(args):
    """One decode step of 16 sequences at position 65536 (summaries of the
    65536 cached tokens precomputed, untimed): hga_decode_step (two launches)
    and hga_route + hga_attend, each replayed as a HIP graph (a serving
    loop's form) and eagerly."""
    import torch
    w = W.DECODE_64K
    pipe = Pipeline(w)
    pipe.build()  # cache + summaries of the 65536 cached tokens and the new token (untimed)
    torch.cuda.synchronize()
    H = pipe.H
    n = max(args.steps * 10, 50)
    nw = max(args.warmup * 10, 50)
    eager_ms, stage = timed_steps(torch, [("route", pipe.route), ("attend", pipe.attend)], n, nw)
    ms_ra = graph_step_ms(torch, [pipe.route, pipe.attend], n, nw)
    ws = H.decode_step_workspace(pipe.cfg, w.batch, w.q_pos0, pipe.q.device)
    lists = H.route_outputs(pipe.cfg, w.batch, w.q_pos0, 1, pipe.q.device)
    out = torch.empty_like(pipe.out)

    def step():
        H.decode_step(pipe.cfg, pipe.q, w.q_pos0, pipe.k_rot, pipe.v, pipe.csum, pipe.gsum, out,
                      None, lists=lists, workspace=ws)
    eager_step_ms, _ = timed_steps(torch, [("decode_step", step)], n, nw)
    ms_step = graph_step_ms(torch, [step], n, nw)
    counts = pipe.ro["granule_count"].cpu().numpy().astype(np.int64)
    bytes_step = decode_bytes(w, counts)
    best = min(ms_step, ms_ra)
    return pipe, dict(us_per_step=best * 1e3,
                      timing="HIP graph replay of one step, the faster of the two paths",
                      decode_step_us=ms_step * 1e3, decode_step_us_eager=eager_step_ms * 1e3,
                      route_attend_us=ms_ra * 1e3, route_attend_us_eager=eager_ms * 1e3,
                      stage_us_eager={k: v * 1e3 for k, v in stage.items()},
                      bytes_per_step=bytes_step, achieved_gbs=bytes_step / (best * 1e-3) / 1e9)


def bench_smalllm(args):
    """The SmallLM-shaped prefill: Mtok/s, and the attention launch against
    the bf16 matrix peak (4 d flops per visible (row, key) pair) and against
    HBM (gathered K and V of the visible tokens plus q and o, 2 bytes each)."""
    import torch
    w = W.SMALLLM_PREFILL
    pipe = Pipeline(w)
    ms, stage = timed_steps(torch, [("build_summaries", pipe.build), ("route", pipe.route),
                                    ("attend", pipe.attend)], args.steps, args.warmup)
    counts = pipe.ro["granule_count"].cpu().numpy()
    pairs = visible_pairs(w, counts)
    flops = 4.0 * w.head_dim * pairs
    keys = int(counts.astype(np.int64).sum()) * w.group_size  # gathered per unit (rows share them)
    gbytes = keys * w.head_dim * 2 * 2 + 2 * w.batch * w.n_q_heads * w.n_q * w.head_dim * 2
    t = stage["attend"] * 1e-3
    return pipe, dict(ms=ms, stage_ms=stage, mtok_s=w.batch * w.n_q / (ms * 1e-3) / 1e6,
                      attend_tflops=flops / t / 1e12, attend_frac_mfma=flops / t / 1e12 / PEAK_BF16_TFLOPS,
                      attend_gathered_bytes=gbytes, attend_gbs=gbytes / t / 1e9,
                      attend_frac_hbm=gbytes / t / 1e9 / PEAK_HBM_GBS)


def bench_tiny(args):
    """The tiny f32 workload (1024 tokens, one head): the whole step's time
    (a launch-latency-bound case)."""
    import torch
    w = W.TINY_F32
    pipe = Pipeline(w)
    ms, stage = timed_steps(torch, [("build_summaries", pipe.build), ("route", pipe.route),
                                    ("attend", pipe.attend)], max(args.steps, 50), max(args.warmup, 20))
    return dict(workload=w.name, us_per_step=ms * 1e3, stage_us={k: v * 1e3 for k, v in stage.items()})


def pinned_copy_gbs(torch, nbytes=256 << 20, reps=5):
    """Measured host->device rate of one large pinned-memory copy."""
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    return nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def bench_host_tier(args, w, copy_gbs, slots=16384, wmax=64, threads=8, cache_slots=0):
    """Prefill with token K/V in pinned host RAM: route + host packing + H2D of
    the routed granules on a side stream + attention, one call per step
    (with a warm tier of cache_slots granules when cache_slots > 0)."""
    import torch
    import hierarchical_kv_routing_amd as H
    pipe = Pipeline(w)
    pipe.build()
    torch.cuda.synchronize()
    # attention alone on device-resident K/V (same granules): the overlap reference
    pipe.route()
    _, st = timed_steps(torch, [("attend", pipe.attend)], 3, 1)
    store = H.host_store(pipe.cfg, pipe.k_rot, pipe.v)
    dev_b, host_b = H.host_tiered_buffer_bytes(pipe.cfg, torch.bfloat16, w.batch, w.q_pos0, w.n_q,
                                               wmax, slots, cache_slots)
    dev = torch.empty(dev_b, dtype=torch.uint8, device="cuda:0")
    host = torch.empty(host_b, dtype=torch.uint8, pin_memory=True)
    lse = torch.empty(pipe.q.shape[:3], dtype=torch.float32, device="cuda:0")
    xs = torch.cuda.Stream()

    def call():
        return H.attend_host_tiered(pipe.cfg, pipe.q, w.q_pos0, store, pipe.k.shape[2], pipe.csum,
                                    pipe.gsum, pipe.out, lse, dev, host, wmax, slots, threads,
                                    copy_stream=xs, cache_slots=cache_slots)

    call()
    torch.cuda.synchronize()
    steps = max(2, min(args.steps, 4))
    t0 = time.perf_counter()
    for _ in range(steps):
        stats = call()
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / steps
    t_copy = stats["bytes_h2d"] / (copy_gbs * 1e9)
    t_attn = st["attend"] * 1e-3
    return dict(workload=w.name, cache_slots=cache_slots, ms=t * 1e3, mtok_s=w.n_q / t / 1e6,
                h2d_gb=stats["bytes_h2d"] / 1e9, h2d_gbs=stats["bytes_h2d"] / t / 1e9,
                pinned_copy_peak_gbs=copy_gbs, windows=stats["windows"],
                granules_copied=stats["granules_copied"], granules_hit=stats["granules_hit"],
                host_pack_s=stats["pack_seconds"], attend_device_ms=st["attend"],
                overlap=(t_copy + t_attn) / t)


STREAM_WARM_STEPS = 64   # one chunk of tokens streamed before the timed session
STREAM_STEPS = 48
STREAM_CACHE_SLOTS = 16384


def bench_stream_decode(args):
    """Decode with the K/V history in pinned host RAM (DecodeSession), one
    token per sequence per step: append (rotate the key, store key and value
    in the host tier, summaries of closed blocks) and step (route, the
    device-side cache lookup, the gather of the misses over the host link,
    attention, all enqueued without a host wait), waited for at the end of
    every step as a serving loop would.  A first
    session streams one chunk of tokens (untimed: first use of the host
    threads and buffers); a second one, started where it ended, with a cold
    device cache, streams the timed steps over new queries."""
    import torch
    import hierarchical_kv_routing_amd as H
    n1, n2 = STREAM_WARM_STEPS, STREAM_STEPS
    prefix = 65536
    w = W.DECODE_64K.scaled(n_ctx=prefix + n1 + n2, kv_cap=prefix + 128, q_pos0=prefix, n_q=n1 + n2)
    pipe = Pipeline(w)
    pipe.build()
    torch.cuda.synchronize()
    cfg = pipe.cfg
    store = H.host_store(cfg, pipe.k_rot, pipe.v)
    store[:, :, prefix // cfg.group_size:] = 0  # the sessions append these tokens
    pipe.csum[:, :, prefix // cfg.chunk_size:] = 0
    pipe.gsum[:, :, prefix // cfg.group_size:] = 0
    cap = pipe.k.shape[2]
    ks = [pipe.k[:, :, p:p + 1].contiguous() for p in range(prefix, prefix + n1 + n2)]
    vs = [pipe.v[:, :, p:p + 1].contiguous() for p in range(prefix, prefix + n1 + n2)]
    qs = [pipe.q[:, :, s:s + 1].contiguous() for s in range(n1 + n2)]
    del pipe.k_rot
    torch.cuda.empty_cache()
    out = torch.empty_like(qs[0])

    def run(first, count):
        sess = H.DecodeSession(cfg, w.batch, cap, prefix + first, STREAM_CACHE_SLOTS, store)
        torch.cuda.synchronize()
        times, stats = [], []
        for s in range(first, first + count):
            pos = prefix + s
            t0 = time.perf_counter()
            sess.append(ks[s], vs[s], pos, pipe.csum, pipe.gsum)
            st = sess.step(qs[s], pos, pipe.csum, pipe.gsum, out, None)
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
            stats.append(st)
        sess.close()
        return np.array(times), stats

    def run_pipelined(first, count):
        # the same steps enqueued back to back (the step does not wait on
        # the host), one wait at the end: a serving loop's steady rate
        sess = H.DecodeSession(cfg, w.batch, cap, prefix + first, STREAM_CACHE_SLOTS, store)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(first, first + count):
            pos = prefix + s
            sess.append(ks[s], vs[s], pos, pipe.csum, pipe.gsum)
            sess.step(qs[s], pos, pipe.csum, pipe.gsum, out, None, stats=False)
        torch.cuda.synchronize()
        total = time.perf_counter() - t0
        sess.close()
        return total / count

    run(0, n1)
    t, stats = run(n1, n2)
    t_pipe = run_pipelined(n1, n2)
    cp = np.array([x["granules_copied"] for x in stats], dtype=np.float64)
    hit = np.array([x["granules_hit"] for x in stats], dtype=np.float64)
    h2d = np.array([x["bytes_h2d"] for x in stats], dtype=np.float64)
    return dict(workload=w.name + "_host_tier_stream", cache_slots=STREAM_CACHE_SLOTS, steps_timed=n2,
                us_per_step_median=float(np.median(t) * 1e6), us_per_step_mean=float(t.mean() * 1e6),
                us_per_step_after_first=float(np.median(t[1:]) * 1e6),
                us_per_step_pipelined=float(t_pipe * 1e6),
                granules_copied_per_step=float(cp[1:].mean()), granules_hit_per_step=float(hit[1:].mean()),
                host_link_mb_per_step=float(h2d[1:].mean() / 1e6),
                first_step_granules_copied=int(cp[0]),
                timing="wall clock of append + step, synchronised every step")


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def _unit_parity(R, p, w, info, gpu_ci, gpu_gi, u):
    """'exact', 'near_tie' or 'mismatch' for one unit's GPU chunk / group
    lists against the oracle's route_unit result (a near-tie: the oracle's
    top-K margin is positive and below 1e-3 |s_(K)|)."""
    g_ch = [int(x) for x in gpu_ci if x >= 0] if p.Kc > 0 else []
    g_gr = [int(x) for x in gpu_gi if x >= 0] if p.Kg > 0 else []
    if g_ch != info["sel_chunks"]:
        return "near_tie" if 0 < info["margin_c"] < 1e-3 * abs(info["s_kc"]) else "mismatch"
    if p.Kg > 0 and g_gr != info["sel_groups"]:
        return "near_tie" if 0 < info["margin_g"] < 1e-3 * abs(info["s_kg"]) else "mismatch"
    return "exact"


def cpu_baseline(pipe, budget_s=12.0):
    """Time the CPU oracle on a bounded, unbiased sample of the prefill step
    and scale to the whole step: summaries of one (sequence, KV head) slab
    and, for randomly ordered units of that slab, routing from those
    summaries and attention over the GPU's own granule lists.  The same
    sample checks the GPU: its routes against the oracle's (exact or
    near-tie) and its outputs against the oracle's attention (exact keys)."""
    from oracle import hga_ref as R
    w = pipe.w
    p = R.params_from_workload(w)
    cores = _blas_threads()
    q, k, v = pipe.q_np, pipe.k_np, pipe.v_np
    t0 = time.time()
    cs, gs = R.summaries(k[0, 0].astype(np.float64), w.n_ctx, p)
    t_sum = time.time() - t0
    csum = np.zeros((1, w.n_kv_heads) + cs.shape)
    gsum = np.zeros((1, w.n_kv_heads) + gs.shape)
    csum[0, 0], gsum[0, 0] = cs, gs
    gr = pipe.ro["granules"].cpu().numpy()
    gc = pipe.ro["granule_count"].cpu().numpy()
    ci = pipe.ro["chunk_idx"].cpu().numpy()
    gi = pipe.ro["group_idx"].cpu().numpy()
    out = pipe.out.float().cpu().numpy()
    nqc = w.n_q // w.chunk_size
    order = np.random.default_rng(0).permutation(nqc)
    done = 0
    tally = dict(exact=0, near_tie=0, mismatch=0)
    diff2 = ref2 = 0.0
    max_abs = 0.0
    t1 = time.time()
    for t in order:
        unit = [(0, 0, int(t))]
        rt = R.route(q, w.q_pos0, w.n_q, csum, gsum, p, units=unit)
        o, _ = R.attend_given(q, w.q_pos0, w.n_q, k, v, gr, gc, p, t0=0, units=unit)
        tally[_unit_parity(R, p, w, rt["info"][unit[0]], ci[0, 0, t], gi[0, 0, t], unit[0])] += 1
        rows = np.s_[0, 0:w.group_ratio, t * w.chunk_size:(t + 1) * w.chunk_size]  # the unit's rows
        dd = out[rows] - o[rows]
        diff2 += float(np.sum(dd * dd))
        ref2 += float(np.sum(o[rows] * o[rows]))
        max_abs = max(max_abs, float(np.abs(dd).max()))
        done += 1
        if time.time() - t1 > budget_s:
            break
    t_units = time.time() - t1
    units_total = w.batch * w.n_kv_heads * nqc
    est_s = t_sum * w.batch * w.n_kv_heads + t_units * units_total / done
    return dict(value=w.n_q / est_s / 1e6, unit="Mtok/s", cores=int(cores), kind="oracle",
                sample=(f"{w.name}: summaries of 1 of {w.batch * w.n_kv_heads} (sequence, kv head) "
                        f"slabs ({t_sum:.2f}s) + route and attention of {done} of {units_total} units "
                        f"in random query-chunk order ({t_units:.2f}s); scaled to the whole step "
                        f"= {est_s:.1f}s per step"),
                parity_on_sample=dict(units=done, routes=tally, attention_max_abs=max_abs,
                                      attention_rel_l2=math.sqrt(diff2 / max(ref2, 1e-300)),
                                      against="the oracle's routes from its own summaries; its "
                                              "attention (exact float64 keys) on the GPU's granule lists"))


def cpu_baseline_decode(pipe, units=4):
    """The oracle on the decode step (one query per (sequence, KV head) unit
    at position 65536): routing from precomputed summaries (untimed, as on
    the GPU) and attention, for a few units, scaled to all 64; parity of
    the GPU's lists and outputs on those units."""
    from oracle import hga_ref as R
    w = pipe.w
    p = R.params_from_workload(w)
    q, k, v = pipe.q_np, pipe.k_np, pipe.v_np
    pick = [(b, h) for b, h in [(0, 0), (5, 2), (11, 1), (15, 3)]][:units]
    t_pos = w.q_pos0 // w.chunk_size
    csum = np.zeros((w.batch, w.n_kv_heads, t_pos + 1, w.head_dim))
    gsum = np.zeros((w.batch, w.n_kv_heads, (t_pos + 1) * (w.chunk_size // w.group_size), w.head_dim))
    for b, h in pick:
        c, g = R.summaries(k[b, h].astype(np.float64), w.n_ctx, p)
        csum[b, h, : c.shape[0]], gsum[b, h, : g.shape[0]] = c, g
    gr = pipe.ro["granules"].cpu().numpy()
    gc = pipe.ro["granule_count"].cpu().numpy()
    ci = pipe.ro["chunk_idx"].cpu().numpy()
    gi = pipe.ro["group_idx"].cpu().numpy()
    out = pipe.out.float().cpu().numpy()
    tally = dict(exact=0, near_tie=0, mismatch=0)
    max_abs = 0.0
    t0 = time.time()
    for b, h in pick:
        unit = [(b, h, t_pos)]
        rt = R.route(q, w.q_pos0, w.n_q, csum, gsum, p, units=unit)
        o, _ = R.attend_given(q, w.q_pos0, w.n_q, k, v, gr, gc, p, t0=t_pos, units=unit)
        tally[_unit_parity(R, p, w, rt["info"][unit[0]], ci[b, h, 0], gi[b, h, 0], unit[0])] += 1
        rows = np.s_[b, h * w.group_ratio:(h + 1) * w.group_ratio, 0]
        max_abs = max(max_abs, float(np.abs(out[rows] - o[rows]).max()))
    t = time.time() - t0
    per_step = t * (w.batch * w.n_kv_heads) / len(pick)
    return dict(value=per_step * 1e6, unit="us/step", cores=_blas_threads(), kind="oracle",
                sample=f"{w.name}: route + attention of {len(pick)} of {w.batch * w.n_kv_heads} units "
                       f"({t:.2f}s), summaries precomputed; scaled to all units",
                parity_on_sample=dict(units=len(pick), routes=tally, attention_max_abs=max_abs))


def cpu_baseline_small(budget_s=4.0):
    """The oracle on the tiny workload (whole step) and the SmallLM-shaped
    prefill (sample, scaled), on all BLAS threads and on one."""
    from oracle import hga_ref as R
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        threadpool_limits = None
    res = {}
    for w in (W.TINY_F32, W.SMALLLM_PREFILL):
        q, k, v = W.make_inputs(w, 0, threads=16)
        p = R.params_from_workload(w)
        nqc = w.n_q // w.chunk_size
        for label, limit in (("all_cores", None), ("one_core", 1)):
            ctx = threadpool_limits(limits=limit) if (limit and threadpool_limits) else None
            if ctx is not None:
                ctx.__enter__()
            try:
                cores = _blas_threads()
                t0 = time.time()
                cs, gs = R.summaries(k[0, 0].astype(np.float64), w.n_ctx, p)
                t_sum = time.time() - t0
                csum = np.zeros((1, 1) + cs.shape)
                gsum = np.zeros((1, 1) + gs.shape)
                csum[0, 0], gsum[0, 0] = cs, gs
                done = 0
                t1 = time.time()
                for t in np.random.default_rng(0).permutation(nqc):
                    unit = [(0, 0, int(t))]
                    rt = R.route(q, w.q_pos0, w.n_q, csum, gsum, p, units=unit)
                    R.attend_given(q, w.q_pos0, w.n_q, k, v, rt["granules"], rt["count"], p, t0=0, units=unit)
                    done += 1
                    if time.time() - t1 > budget_s:
                        break
                t_units = time.time() - t1
            finally:
                if ctx is not None:
                    ctx.__exit__(None, None, None)
            slabs = w.batch * w.n_kv_heads
            est = t_sum * slabs + t_units * slabs * nqc / done
            res[f"{w.name}:{label}"] = dict(value=w.batch * w.n_q / est / 1e6, unit="Mtok/s", cores=cores,
                                            kind="oracle", seconds_per_step=est,
                                            sample=f"{done} of {slabs * nqc} units timed, scaled")
    return res


def copy_calibration(args):
    """A plain device copy of known size (for scaling HBM byte counters)."""
    import torch
    n = 1 << 28  # 256 Mi bf16 elements = 512 MiB
    a = torch.empty(n, dtype=torch.bfloat16, device="cuda:0").normal_()
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {2 * n} bytes read and written per launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "smalllm", "tiny", "host", "stream", "backward",
                                       "copy", "peaks"], default=None)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the routed-attention hot path runs per (sequence, KV head) unit on one device "
              "and this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import hierarchical_kv_routing_amd as H
    H.lib()

    if args.only == "copy":
        copy_calibration(args)
        return
    if args.only == "peaks":
        print(json.dumps(dict(peaks_measured=measured_peaks(torch))), flush=True)
        return
    if args.only == "decode":
        _, dec = bench_decode(args)
        print(json.dumps(dict(decode=dec)), flush=True)
        return
    if args.only == "tiny":
        print(json.dumps(dict(tiny=bench_tiny(args))), flush=True)
        return
    if args.only == "host":
        gbs = pinned_copy_gbs(torch)
        res = {w.name + ("" if c == 0 else "_warm_tier"): bench_host_tier(args, w, gbs, cache_slots=c)
               for w in (W.HOST_TIERED_CHUNK, W.HOST_TIERED_GROUP) for c in (0, WARM_TIER_SLOTS)}
        print(json.dumps(dict(host_tiered=res)), flush=True)
        return
    if args.only == "backward":
        print(json.dumps(dict(backward=bench_backward(args))), flush=True)
        return
    if args.only == "stream":
        print(json.dumps(dict(decode_host_tier_stream=bench_stream_decode(args))), flush=True)
        return
    if args.only == "smalllm":
        _, sm = bench_smalllm(args)
        print(json.dumps(dict(smalllm=sm)), flush=True)
        return

    pipe, pre = bench_prefill(args)
    log(f"[bench] prefill: {pre['ms']:.3f} ms/step, stages {pre['stage_ms']}")
    w = pipe.w
    value = pre["tokens"] / (pre["ms"] * 1e-3) / 1e6
    line = dict(
        metric=METRIC, value=value, unit="Mtok/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=pre["ms"], higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16", data="synthetic",
        config=dict(workload=w.name, batch=w.batch, seq_len=w.n_ctx, q_heads=w.n_q_heads,
                    kv_heads=w.n_kv_heads, head_dim=w.head_dim, C=w.chunk_size, g_s=w.group_size,
                    F=w.n_sink_chunks, L=w.n_recent_chunks, K_c=w.top_chunks, K_g=w.top_groups,
                    rope_theta=w.rope_theta),
        roofline=dict(bound="mfma", kernel="attend_mfma_kernel", achieved=pre["attend_tflops"],
                      peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                      frac=pre["attend_tflops"] / PEAK_BF16_TFLOPS, traffic=recorded_traffic(),
                      traffic_unit="bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE)",
                      flops_per_launch=pre["attend_flops"], visible_pairs=pre["pairs"],
                      avg_launch_ms=pre["stage_ms"]["attend"]),
        stage_ms=pre["stage_ms"],
    )
    if args.only is None:
        peaks = measured_peaks(torch)
        line["peaks_measured"] = peaks
        line["roofline"]["frac_of_measured_peak"] = pre["attend_tflops"] / peaks["mfma_bf16_tflops"]
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline(pipe)
            log(f"[bench] cpu baseline: {line['cpu_baseline']}")
        line["backward"] = bench_backward(args, pipe, pre["pairs"])
        log(f"[bench] backward: {line['backward']}")
        del pipe
        torch.cuda.empty_cache()
        dpipe, dec = bench_decode(args)
        line["decode"] = dict(workload=W.DECODE_64K.name, **{k: v for k, v in dec.items()
                                                             if k not in ("bytes_per_step", "achieved_gbs")},
                              roofline=dict(bound="hbm", achieved=dec["achieved_gbs"], peak=PEAK_HBM_GBS,
                                            unit="GB/s", frac=dec["achieved_gbs"] / PEAK_HBM_GBS,
                                            frac_of_measured_peak=dec["achieved_gbs"] / peaks["hbm_copy_gbs"],
                                            bytes_per_step=dec["bytes_per_step"]))
        if not args.no_cpu_baseline:
            line["decode"]["cpu_baseline"] = cpu_baseline_decode(dpipe)
        log(f"[bench] decode: {line['decode']}")
        del dpipe
        torch.cuda.empty_cache()
        _, sm = bench_smalllm(args)
        line["smalllm"] = dict(workload=W.SMALLLM_PREFILL.name, **sm)
        line["tiny"] = bench_tiny(args)
        if not args.no_cpu_baseline:
            line["cpu_baseline_small"] = cpu_baseline_small()
        torch.cuda.empty_cache()
        gbs = pinned_copy_gbs(torch)
        line["host_tiered"] = {}
        for w in (W.HOST_TIERED_CHUNK, W.HOST_TIERED_GROUP):
            for cache in (0, WARM_TIER_SLOTS):
                name = w.name + ("" if cache == 0 else "_warm_tier")
                line["host_tiered"][name] = bench_host_tier(args, w, gbs, cache_slots=cache)
                log(f"[bench] host tier {name}: {line['host_tiered'][name]}")
                torch.cuda.empty_cache()
        line["decode_host_tier_stream"] = bench_stream_decode(args)
        log(f"[bench] streaming decode from the host tier: {line['decode_host_tier_stream']}")
        torch.cuda.empty_cache()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
