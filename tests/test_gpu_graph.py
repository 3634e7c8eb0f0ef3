"""GPU test: a decode step (route + attend) captured as one HIP graph and
replayed gives the eager results bit for bit on every replay, with eager
work and synchronizations between the replays."""
import pytest

import hierarchical_kv_routing_amd as H
import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("batch", [3, 16])  # segmented scoring / one workgroup per unit
def test_decode_step_graph_replays_match_eager(batch):
    import torch
    w = W.DECODE_64K.scaled(batch=batch, n_ctx=20481, kv_cap=20544, q_pos0=20480)
    q, k, v = P.make_inputs_parallel(w)
    run = P.GpuRun(w, q, k, v)
    ro, cfg = run.ro, run.cfg
    out = torch.empty_like(run.out)
    lse = torch.empty_like(run.lse)
    ws = torch.empty(max(H.attend_workspace_bytes(cfg, w.batch, w.q_pos0, w.n_q), 16),
                     dtype=torch.uint8, device="cuda:0")

    def step():
        H.route(cfg, run.q, w.q_pos0, run.csum, run.gsum, run.k.shape[2], ro["chunk_idx"],
                ro["group_idx"], ro["granules"], ro["granule_count"], ro["workspace"])
        H.attend(cfg, run.q, w.q_pos0, run.k_rot, run.v, ro["granules"], ro["granule_count"],
                 out, lse, ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (ro["granules"], ro["granule_count"], out, lse)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (ro["granules"], out, lse):
            t.fill_(-7) if t.dtype == torch.int32 else t.fill_(float("nan"))
        ro["granule_count"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (ro["granules"], ro["granule_count"], out, lse)
        same = [bool(torch.equal(a, b)) for a, b in zip(got, ref)]
        print(f"[gpu] graph replay {rep} batch {batch}: {same}", flush=True)
        assert all(same), (rep, same)
        _ = (run.q.float() * 2).sum().item()  # eager work between replays
