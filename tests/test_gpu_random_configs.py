"""GPU parity over seeded random shapes (tests/random_configs.py): summaries
of one slab, every unit's routes (exact up to near-ties) and attention on
the GPU's granule lists, against the CPU fp64 oracle, for each drawn mix of
chunk / group size, windows, budgets, GQA ratio, head size, dtype, ragged
start and RoPE wrap."""
import pytest

import hierarchical_kv_routing_amd as H
from oracle import hga_ref as R
from tests import parity as P
from tests.random_configs import N_CONFIGS, N_DECODE, random_decode_workload, random_workload


@pytest.mark.parametrize("i", range(N_CONFIGS + N_DECODE))
def test_random_shape_accepted(i):
    """Every drawn shape is inside the library's limits (CPU: sizing calls only)."""
    w = random_workload(i) if i < N_CONFIGS else random_decode_workload(i - N_CONFIGS)
    cfg = H.Config.from_workload(w)
    assert 0 < H.max_granules(cfg) <= 2048
    assert H.route_workspace_bytes(cfg, w.batch, w.q_pos0, w.n_q) >= 0
    assert H.attend_workspace_bytes(cfg, w.batch, w.q_pos0, w.n_q) >= 0


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CONFIGS))
def test_random_shape_parity(i):
    w = random_workload(i)
    print(f"[gpu] random shape {i}: {w}", flush=True)
    q, k, v = P.make_inputs_parallel(w, seed=i)
    run = P.DeviceRun(w, q, k, v)
    P.check_summaries(run, k, slabs=[(w.batch - 1, w.n_kv_heads - 1)])
    units = P.all_units(w)
    orc = P.oracle_route(run, q, k, units)
    exact, near = P.compare_routes(run, orc, units)
    assert exact + near == len(units)
    assert near <= max(2, len(units) // 50)
    P.check_attention(run, q, k, v, units)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_DECODE))
def test_random_decode_parity(i):
    w = random_decode_workload(i)
    print(f"[gpu] random decode {i}: {w}", flush=True)
    q, k, v = P.make_inputs_parallel(w, seed=i)
    run = P.DeviceRun(w, q, k, v)
    P.check_summaries(run, k, slabs=[(w.batch - 1, w.n_kv_heads - 1)])
    units = P.all_units(w)
    orc = P.oracle_route(run, q, k, units)
    exact, near = P.compare_routes(run, orc, units)
    assert exact + near == len(units)
    assert near <= max(1, len(units) // 20)
    P.check_attention(run, q, k, v, units)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(1, N_CONFIGS, 4))
def test_random_shape_dense_and_full_coverage(i):
    """Eq. 1 on random shapes: hga_dense_causal, and routing whose chunk
    budget covers every middle chunk (K_g = 0), both against the oracle's
    dense causal attention over every query row."""
    import torch
    w0 = random_workload(i)
    w = w0.scaled(top_chunks=w0.kv_cap // w0.chunk_size, top_groups=0)
    print(f"[gpu] random dense {i}: {w}", flush=True)
    q, k, v = P.make_inputs_parallel(w, seed=i)
    run = P.DeviceRun(w, q, k, v)
    dense = torch.full_like(run.out, float("nan"))
    dlse = torch.full_like(run.lse, float("nan"))
    H.dense_causal(run.cfg, run.q, w.q_pos0, run.k_rot, run.v, dense, dlse, run.aws)
    torch.cuda.synchronize()
    P.check_dense(w, dense.float().cpu().numpy(), dlse.cpu().numpy(), q, k, v, name=f"random{i}:dense")
    P.check_dense(w, run.np("out"), run.np("lse"), q, k, v, name=f"random{i}:full_coverage")
