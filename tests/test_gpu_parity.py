"""GPU parity: every step of the HIP path vs the CPU fp64 oracle.

Sizes are chosen so the oracle finishes in seconds while each call still
spans many tiles and a ragged tail (context not a multiple of the chunk).
Tolerances and the near-tie rule are stated in tests/parity.py.
"""
import numpy as np
import pytest

import hierarchical_kv_routing_amd as H
import workloads as W
from oracle import hga_ref as R
from tests import parity as P

pytestmark = pytest.mark.gpu


def _small(base, **kw):
    return base.scaled(**kw)


# Oracle-sized versions of the five workloads (same head shapes, budgets and
# distributions; shorter contexts with ragged tails).
CASES = {
    "tiny_f32": W.TINY_F32,
    "smalllm_ragged": _small(W.SMALLLM_PREFILL, batch=2, n_q_heads=4, n_kv_heads=4,
                             n_ctx=1000, kv_cap=1024, n_q=1000, planted=8),
    "qwen3_ragged": _small(W.QWEN3_PREFILL, n_ctx=2500, kv_cap=2560, n_q=2500, planted=16),
    "qwen3_chunk_only": _small(W.HOST_TIERED_CHUNK, n_ctx=3000, kv_cap=3008, n_q=3000, planted=16),
    "qwen3_group_k16": _small(W.HOST_TIERED_GROUP, n_ctx=3000, kv_cap=3008, n_q=3000, planted=16),
}


def _inputs(w, seed=0):
    return P.make_inputs_parallel(w, seed)


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    w = CASES[request.param]
    q, k, v = _inputs(w)
    print(f"[gpu] case {request.param}: {w}", flush=True)
    run = P.DeviceRun(w, q, k, v)
    return request.param, w, q, k, v, run


def test_summaries_and_rotated_keys(case):
    name, w, q, k, v, run = case
    P.check_summaries(run, k)


def test_routes(case):
    name, w, q, k, v, run = case
    units = P.all_units(w)
    orc = P.oracle_route(run, q, k, units)
    exact, near = P.compare_routes(run, orc, units)
    print(f"[gpu] {name}: routes exact={exact} near_tie={near} of {len(units)}", flush=True)
    assert near <= max(2, len(units) // 50)


def test_attention(case):
    name, w, q, k, v, run = case
    units = P.all_units(w)
    m, r, l = P.check_attention(run, q, k, v, units)
    print(f"[gpu] {name}: attention max_abs={m:.3g} rel_l2={r:.3g} lse={l:.3g}", flush=True)


def test_deterministic(case):
    name, w, q, k, v, run = case
    out0, gr0 = run.np("out"), run.np("granules")
    run.route()
    run.attend()
    import torch
    torch.cuda.synchronize()
    assert np.array_equal(run.np("granules"), gr0)
    assert np.array_equal(run.np("out"), out0)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_full_coverage_equals_dense(dtype, d):
    """Budgets covering every middle chunk: routed attention equals dense
    causal attention (Eq. 1), on the GPU bit for bit and against the oracle."""
    w = _small(W.QWEN3_PREFILL, dtype=dtype, head_dim=d, n_q_heads=8, n_kv_heads=2,
               n_ctx=1280, kv_cap=1280, n_q=1280, top_chunks=64, top_groups=0,
               n_hf_pairs=R.high_freq_pair_count(d, 1e7, 64), planted=4)
    q, k, v = _inputs(w, seed=1)
    run = P.DeviceRun(w, q, k, v)
    import torch
    dense = torch.zeros_like(run.out)
    dlse = torch.zeros_like(run.lse)
    H.dense_causal(run.cfg, run.q, 0, run.k_rot, run.v, dense, dlse, run.aws)
    torch.cuda.synchronize()
    same_out = bool(torch.equal(dense, run.out))
    assert same_out, "routed full coverage differs from dense"
    same_lse = bool(torch.equal(dlse, run.lse))
    assert same_lse, "routed full coverage LSE differs from dense"
    heads = [0, 5]
    qi = np.r_[0:70, 600:640, 1200:1280]
    P.check_dense(w, run.np("out"), run.np("lse"), q, k, v, heads=heads, q_index=qi)


def test_dense_causal_partial_queries():
    """Dense path with q_pos0 inside a chunk and a ragged end."""
    w = _small(W.SMALLLM_PREFILL, batch=1, n_q_heads=2, n_kv_heads=1, n_ctx=700, kv_cap=704,
               q_pos0=133, n_q=567, planted=0)
    q, k, v = _inputs(w, seed=2)
    run = P.DeviceRun(w, q, k, v, route=False, attend=False)
    import torch
    H.dense_causal(run.cfg, run.q, w.q_pos0, run.k_rot, run.v, run.out, run.lse, run.aws)
    torch.cuda.synchronize()
    P.check_dense(w, run.np("out"), run.np("lse"), q, k, v)


EDGE = {
    "no_routing_kc0": dict(top_chunks=0, top_groups=0),
    "chunk_only": dict(top_groups=0),
    "no_recent_no_sink": dict(n_recent_chunks=0, n_sink_chunks=0),
    "granule_is_chunk": dict(group_size=64, top_groups=3),
    "group_size_8": dict(group_size=8, top_groups=24),
    "ragged_start": dict(q_pos0=200, n_q=811),
    "single_query_at_0": dict(q_pos0=0, n_q=1),
    "budget_above_candidates": dict(top_chunks=200, top_groups=250),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_cases(name):
    over = dict(n_ctx=1011, kv_cap=1024, n_q=1011, planted=8)
    over.update(EDGE[name])
    w = _small(W.QWEN3_PREFILL, **over)
    q, k, v = _inputs(w, seed=3)
    run = P.DeviceRun(w, q, k, v)
    units = P.all_units(w)
    orc = P.oracle_route(run, q, k, units)
    P.compare_routes(run, orc, units)
    P.check_attention(run, q, k, v, units)


# Wrapped RoPE positions (xllm-io page, Sec. 5.5 variant; period a multiple
# of C).  Small periods make oracle-sized contexts wrap several times; the f32
# case runs the f32 attention kernel, the ragged start a unit that begins
# mid-chunk, and the decode case a query whose wrapped position is 0.
WRAP = {
    "f32_tiny_p256": _small(W.TINY_F32, rope_period=256),
    "qwen3_ragged_p512": _small(W.QWEN3_PREFILL, n_ctx=2500, kv_cap=2560, n_q=2500, planted=16,
                                rope_period=512),
    "qwen3_ragged_start_p192": _small(W.QWEN3_PREFILL, n_ctx=1011, kv_cap=1024, q_pos0=200,
                                      n_q=811, planted=8, rope_period=192),
    "decode_p4096": _small(W.DECODE_64K, batch=3, n_ctx=20481, kv_cap=20544, q_pos0=20480,
                           rope_period=4096),
}


@pytest.mark.parametrize("name", sorted(WRAP))
def test_rope_wrap(name):
    w = WRAP[name]
    q, k, v = _inputs(w, seed=5)
    print(f"[gpu] rope wrap {name}: {w}", flush=True)
    run = P.DeviceRun(w, q, k, v)
    P.check_summaries(run, k, slabs=[(0, 0), (w.batch - 1, w.n_kv_heads - 1)])
    units = P.all_units(w)
    orc = P.oracle_route(run, q, k, units)
    exact, near = P.compare_routes(run, orc, units)
    assert near <= max(2, len(units) // 50)
    P.check_attention(run, q, k, v, units)
    # the period reaches the kernels: absolute positions give other outputs
    flat = P.DeviceRun(w.scaled(rope_period=0), q, k, v)
    assert not np.array_equal(flat.np("out"), run.np("out"))


def test_empty_call_is_noop():
    w = _small(W.SMALLLM_PREFILL, batch=1, n_q_heads=1, n_kv_heads=1, n_ctx=128, kv_cap=128,
               n_q=128, planted=0)
    q, k, v = _inputs(w)
    run = P.DeviceRun(w, q, k, v)
    import torch
    before = run.out.clone()
    H.attend(run.cfg, run.q[:, :, :0], 0, run.k_rot, run.v, run.ro["granules"][:, :, :0],
             run.ro["granule_count"][:, :, :0], run.out[:, :, :0].contiguous(), None, run.aws)
    torch.cuda.synchronize()
    same = bool(torch.equal(before, run.out))
    assert same, "empty call wrote the output"


def test_summary_single_token_blocks():
    """C = g_s = 1: every summary equals the rotated key (GPU vs its own k_rot
    and vs the oracle)."""
    w = _small(W.TINY_F32, chunk_size=1, group_size=1, n_ctx=256, kv_cap=256, n_q=256,
               n_hf_pairs=5, planted=0)
    q, k, v = _inputs(w)
    run = P.DeviceRun(w, q, k, v, route=False, attend=False)
    P.check_summaries(run, k)
    np.testing.assert_allclose(run.np("csum")[0, 0], run.np("k_rot")[0, 0], atol=1e-6)
    np.testing.assert_allclose(run.np("gsum")[0, 0], run.np("k_rot")[0, 0], atol=1e-6)


def test_append_matches_prefill_build():
    """Appending tokens one at a time (the decode append of a closed chunk)
    gives the same cache and summaries as one prefill build (the pages'
    cache vs no-cache check)."""
    w = _small(W.QWEN3_PREFILL, n_ctx=700, kv_cap=704, n_q=700, planted=0)
    q, k, v = _inputs(w)
    full = P.DeviceRun(w, q, k, v, route=False, attend=False)
    inc = P.DeviceRun(w, q, k, v, build=False, route=False, attend=False)
    import torch
    H.build_summaries(inc.cfg, inc.k, 0, 500, inc.k_rot, inc.csum, inc.gsum)
    for p in range(500, 700):
        H.build_summaries(inc.cfg, inc.k, p, p + 1, inc.k_rot, inc.csum, inc.gsum)
    torch.cuda.synchronize()
    same = [bool(torch.equal(getattr(full, n), getattr(inc, n))) for n in ("k_rot", "csum", "gsum")]
    assert all(same), same


def test_decode_segmented_and_split():
    """Decode-shaped call (one query per sequence, long context): segmented
    chunk scoring and split-key attention with the partial merge."""
    w = _small(W.DECODE_64K, batch=3, n_ctx=20481, kv_cap=20544, q_pos0=20480)
    q, k, v = _inputs(w)
    cfg = H.Config.from_workload(w)
    assert H.route_workspace_bytes(cfg, w.batch, w.q_pos0, 1) > 0
    assert H.attend_workspace_bytes(cfg, w.batch, w.q_pos0, 1) > 0
    run = P.DeviceRun(w, q, k, v)
    units = P.all_units(w)
    P.check_summaries(run, k, slabs=[(0, 0), (2, 3)])
    orc = P.oracle_route(run, q, k, units)
    exact, near = P.compare_routes(run, orc, units)
    assert exact + near == len(units)
    P.check_attention(run, q, k, v, units)
