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
    run = P.DeviceRun(w, q, k, v)
    P.check_summaries(run, k, slabs=[(0, 0), (0, 3)])
    units = P.all_units(w)
    orc = P.oracle_route(run, q, k, units)
    exact, near = P.compare_routes(run, orc, units, name="fullsize:" + w.name)
    print(f"[gpu] qwen3 32k routes: exact={exact} near_tie={near} of {len(units)}", flush=True)
    assert near <= len(units) // 50
    last = w.n_q // w.chunk_size - 1
    att = sorted(set(P.sample_units(w, 256)) | {(0, h, last) for h in range(w.n_kv_heads)})
    m, r, l = P.check_attention(run, q, k, v, att, name="fullsize:" + w.name)
    print(f"[gpu] qwen3 32k attention on {len(att)} units: max_abs={m:.3g} rel_l2={r:.3g}", flush=True)


def test_smalllm_prefill_4k_full():
    """The SmallLM-shaped prefill bench.py also times (4 sequences, 8 / 8
    heads, d = 64, 4096 tokens): every unit's routes, the attention of
    every row of sampled units."""
    w = W.SMALLLM_PREFILL
    q, k, v = P.make_inputs_parallel(w)
    run = P.DeviceRun(w, q, k, v)
    P.check_summaries(run, k, slabs=[(0, 0), (3, 7)])
    units = P.all_units(w)
    orc = P.oracle_route(run, q, k, units)
    exact, near = P.compare_routes(run, orc, units, name="fullsize:" + w.name)
    print(f"[gpu] smalllm 4k routes: exact={exact} near_tie={near} of {len(units)}", flush=True)
    assert near <= len(units) // 50
    m, r, l = P.check_attention(run, q, k, v, P.sample_units(w, 256), name="fullsize:" + w.name)
    print(f"[gpu] smalllm 4k attention: max_abs={m:.3g} rel_l2={r:.3g}", flush=True)


def test_decode_64k_full():
    w = W.DECODE_64K
    q, k, v = P.make_inputs_parallel(w)
    print("[gpu] decode 64k: inputs ready", flush=True)
    run = P.DeviceRun(w, q, k, v)
    units = P.all_units(w)          # all 64 (sequence, KV head) units
    P.check_summaries(run, k, slabs=[(0, 0), (5, 2), (11, 1), (15, 3)])
    orc = P.oracle_route(run, q, k, units)
    exact, near = P.compare_routes(run, orc, units, name="fullsize:" + w.name)
    print(f"[gpu] decode 64k routes: exact={exact} near_tie={near} of {len(units)}", flush=True)
    assert exact + near == len(units)
    m, r, l = P.check_attention(run, q, k, v, units, name="fullsize:" + w.name)
    print(f"[gpu] decode 64k attention on {len(units)} units: max_abs={m:.3g} rel_l2={r:.3g}", flush=True)


# "group_wrap64k": RoPE positions wrapped modulo 65536 (xllm-io page,
# Sec. 5.5 variant) over 131072 tokens, through the warm tier (a device
# cache of 8192 granules), so the second half of the sequence rotates as
# the first.
@pytest.mark.parametrize("base", ["chunk_only", "group", "group_wrap64k"])
def test_host_tiered_128k_full(base):
    import torch
    w = {"chunk_only": W.HOST_TIERED_CHUNK, "group": W.HOST_TIERED_GROUP,
         "group_wrap64k": W.HOST_TIERED_GROUP.scaled(rope_period=65536)}[base]
    cache = 8192 if w.rope_period else 0
    q, k, v = P.make_inputs_parallel(w)
    print(f"[gpu] host tier 128k {base}: inputs ready", flush=True)
    run = P.DeviceRun(w, q, k, v)
    slots = 16384
    if w.rope_period:
        P.check_summaries(run, k, slabs=[(0, 2)])
    out, lse, stats = run_host_tier(run, max_window_chunks=64, slots=slots, threads=8,
                                    cache_slots=cache)
    print(f"[gpu] host tier 128k {base}: {stats}", flush=True)
    same = bool(torch.equal(out, run.out))
    assert same, "host tier differs from the device-resident path"
    # 64 units spread over the query chunks and KV heads, with the last chunk
    nqc = w.n_q // w.chunk_size
    units = sorted({(0, i % w.n_kv_heads, int(t)) for i, t in enumerate(np.linspace(11, nqc - 1, 64))}
                   | {(0, 3, nqc - 1)})
    orc = P.oracle_route(run, q, k, units)
    exact, near = P.compare_routes(run, orc, units, name=f"fullsize:{base}")
    print(f"[gpu] host tier 128k {base}: routes exact={exact} near_tie={near} of {len(units)}", flush=True)
    P.check_attention(run, q, k, v, units, out=out.float().cpu().numpy(), lse=lse.cpu().numpy(),
                      name=f"fullsize:{base}")
