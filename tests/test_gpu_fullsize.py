"""Parity at the full workload sizes, in the launch configuration bench.py
times.  The oracle checks every unit's routing where that is cheap (the
32768-token prefill) and samples units elsewhere; attention is checked on
sampled units computed one by one from the GPU's granule lists."""
import numpy as np
import pytest

import hierarchical_kv_routing_amd as H
import workloads as W
from tests import parity as P
from tests.test_gpu_host_tier import run_host_tier

pytestmark = pytest.mark.gpu


def test_qwen3_prefill_32k_full():
    w = W.QWEN3_PREFILL
    q, k, v = P.make_inputs_parallel(w)
    print("[gpu] qwen3 prefill 32k: inputs ready", flush=True)
    run = P.GpuRun(w, q, k, v)
    P.check_summaries(run, k, slabs=[(0, 0), (0, 3)])
    units = P.all_units(w)
    orc = P.oracle_route(run, q, k, units)
    exact, near = P.compare_routes(run, orc, units)
    print(f"[gpu] qwen3 32k routes: exact={exact} near_tie={near} of {len(units)}", flush=True)
    assert near <= len(units) // 50
    m, r, l = P.check_attention(run, q, k, v, P.sample_units(w, 12))
    print(f"[gpu] qwen3 32k attention: max_abs={m:.3g} rel_l2={r:.3g}", flush=True)


def test_decode_64k_full():
    w = W.DECODE_64K
    q, k, v = P.make_inputs_parallel(w)
    print("[gpu] decode 64k: inputs ready", flush=True)
    run = P.GpuRun(w, q, k, v)
    units = [(0, 0, 1024), (5, 2, 1024), (11, 1, 1024), (15, 3, 1024)]
    P.check_summaries(run, k, slabs=[(b, h) for b, h, _ in units])
    orc = P.oracle_route(run, q, k, units)
    exact, near = P.compare_routes(run, orc, units)
    assert exact + near == len(units)
    P.check_attention(run, q, k, v, units)


@pytest.mark.parametrize("base", ["chunk_only", "group"])
def test_host_tiered_128k_full(base):
    import torch
    w = W.HOST_TIERED_CHUNK if base == "chunk_only" else W.HOST_TIERED_GROUP
    q, k, v = P.make_inputs_parallel(w)
    print(f"[gpu] host tier 128k {base}: inputs ready", flush=True)
    run = P.GpuRun(w, q, k, v)
    slots = 16384
    out, lse, stats = run_host_tier(run, max_window_chunks=64, slots=slots, threads=8)
    print(f"[gpu] host tier 128k {base}: {stats}", flush=True)
    same = bool(torch.equal(out, run.out))
    assert same, "host tier differs from the device-resident path"
    units = [(0, 0, 2047), (0, 3, 1500), (0, 1, 700)]
    orc = P.oracle_route(run, q, k, units)
    P.compare_routes(run, orc, units)
    P.check_attention(run, q, k, v, units, out=out.float().cpu().numpy(), lse=lse.cpu().numpy())
