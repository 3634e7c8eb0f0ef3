"""GPU parity of hga_decode_step (one decode step in two launches) against
the oracle: routes bit-exact except counted near-ties, attention within the
tolerances of tests/parity.py on the step's own granule lists; at the full
decode workload (16 sequences x 4 KV heads at position 65536) on every unit,
on the random decode shapes and on edge cases.  Also: repeated calls on a
workspace full of NaN bits and HIP graph replays give the same bits, and
skipping the lists leaves the output unchanged."""
import numpy as np
import pytest

import hierarchical_kv_routing_amd as H
import workloads as W
from tests import parity as P
from tests.random_configs import N_DECODE, random_decode_workload

pytestmark = pytest.mark.gpu


class StepRun(P.DeviceRun):
    """DeviceRun whose routes and attention come from hga_decode_step."""

    def __init__(self, w, q, k, v, cfg=None):
        import torch
        super().__init__(w, q, k, v, cfg=cfg, route=False, attend=False)
        self.ws = H.decode_step_workspace(self.cfg, w.batch, w.q_pos0, self.q.device)
        self.ws.fill_(255)  # the step may not rely on the workspace's contents
        self.step()
        torch.cuda.synchronize()

    def step(self, lists=True, out=None, lse=None):
        H.decode_step(self.cfg, self.q, self.w.q_pos0, self.k_rot, self.v, self.csum, self.gsum,
                      self.out if out is None else out, self.lse if lse is None else lse,
                      lists=self.ro if lists else None, workspace=self.ws)


def _check(w, seed=0, name=None, k_edit=None):
    q, k, v = P.make_inputs_parallel(w, seed)
    if k_edit is not None:
        k = k_edit(k)
    run = StepRun(w, q, k, v)
    units = P.all_units(w)
    orc = P.oracle_route(run, q, k, units)
    exact, near = P.compare_routes(run, orc, units, name=f"decode_step:{name or w.name}")
    assert exact + near == len(units)
    m, r, _ = P.check_attention(run, q, k, v, units, name=f"decode_step:{name or w.name}")
    print(f"[gpu] decode_step {name or w.name}: routes exact={exact} near={near}; "
          f"max_abs={m:.3g} rel_l2={r:.3g}", flush=True)
    return run


def test_decode_step_full_64k():
    """The decode workload as bench.py times it: all 64 units."""
    w = W.DECODE_64K
    print(f"[gpu] decode_step full: {w}", flush=True)
    run = _check(w, name="full_64k")
    # a second call on the same workspace: bitwise the same
    import torch
    out2 = torch.full_like(run.out, float("nan"))
    lse2 = torch.full_like(run.lse, float("nan"))
    run.step(out=out2, lse=lse2)
    torch.cuda.synchronize()
    assert torch.equal(out2, run.out) and torch.equal(lse2, run.lse)


@pytest.mark.parametrize("i", range(N_DECODE))
def test_decode_step_random_shapes(i):
    w = random_decode_workload(i)
    cfg = H.Config.from_workload(w)
    if H.decode_step_workspace_bytes(cfg, w.batch, w.q_pos0) == 0:
        pytest.skip("shape outside hga_decode_step's limits (hga_route + hga_attend cover it)")
    print(f"[gpu] decode_step random {i}: {w}", flush=True)
    _check(w, seed=i, name=f"random_decode_{i}")


_BASE = W.DECODE_64K.scaled(batch=3, n_ctx=12289, kv_cap=12352, q_pos0=12288)
EDGE = {
    "no_routing_kc0": _BASE.scaled(top_chunks=0, top_groups=0),
    "chunk_only": _BASE.scaled(top_groups=0),
    "gqa1": _BASE.scaled(n_q_heads=4),
    "gqa16": _BASE.scaled(n_q_heads=64),
    "d64": _BASE.scaled(head_dim=64, rope_theta=1e4, n_hf_pairs=9),
    "pos_mid_chunk": _BASE.scaled(n_ctx=12320, q_pos0=12319),
    "few_chunks": _BASE.scaled(n_ctx=700, kv_cap=704, q_pos0=699),
    "inside_fixed_windows": _BASE.scaled(n_ctx=300, kv_cap=320, q_pos0=299),
    "first_token": _BASE.scaled(n_ctx=1, kv_cap=64, q_pos0=0),
    "rope_wrap": _BASE.scaled(rope_period=4096),
    "budget_above_candidates": _BASE.scaled(n_ctx=1300, kv_cap=1344, q_pos0=1299, top_chunks=200,
                                            top_groups=250),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_decode_step_edge_cases(name):
    w = EDGE[name]
    print(f"[gpu] decode_step edge {name}: {w}", flush=True)
    _check(w, seed=5, name=name)


def test_decode_step_exact_ties():
    """Zero keys in every middle chunk but three: the lowest index wins the
    tied places, across the scan items' segments."""
    w = W.DECODE_64K.scaled(batch=2, n_ctx=32769, kv_cap=32832, q_pos0=32768, planted_per_q_head=0)

    def zero(k):
        C = w.chunk_size
        keep = np.zeros(w.kv_cap // C, bool)
        keep[: w.n_sink_chunks] = True
        keep[[20, 100, 300]] = True
        k = k.reshape(w.batch, w.n_kv_heads, -1, C, w.head_dim).copy()
        k[:, :, ~keep] = 0.0
        return k.reshape(w.batch, w.n_kv_heads, w.kv_cap, w.head_dim)
    _check(w, seed=3, name="exact_ties", k_edit=zero)


def test_decode_step_without_lists_same_output():
    import torch
    w = _BASE
    q, k, v = P.make_inputs_parallel(w, 2)
    run = StepRun(w, q, k, v)
    out2 = torch.full_like(run.out, float("nan"))
    lse2 = torch.full_like(run.lse, float("nan"))
    run.step(lists=False, out=out2, lse=lse2)
    torch.cuda.synchronize()
    assert torch.equal(out2, run.out) and torch.equal(lse2, run.lse)


def test_decode_step_graph_replays_match_eager():
    """The step captured as a HIP graph: every replay (eager work and
    synchronizations between them) gives the eager bits."""
    import torch
    w = W.DECODE_64K.scaled(n_ctx=20481, kv_cap=20544, q_pos0=20480)
    q, k, v = P.make_inputs_parallel(w)
    run = StepRun(w, q, k, v)
    ref = [t.clone() for t in (run.ro["granules"], run.ro["granule_count"], run.out, run.lse)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.step()
    for rep in range(3):
        run.ro["granules"].fill_(-7)
        run.ro["granule_count"].fill_(-7)
        run.out.fill_(float("nan"))
        run.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (run.ro["granules"], run.ro["granule_count"], run.out, run.lse)
        same = [bool(torch.equal(a, b)) for a, b in zip(got, ref)]
        print(f"[gpu] decode_step graph replay {rep}: {same}", flush=True)
        assert all(same), (rep, same)
        _ = (run.q.float() * 2).sum().item()
