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
    run = P.DeviceRun(w, q, k, v)
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


@pytest.mark.parametrize("shape", ["qwen3", "smalllm"])  # split-table routing / direct scoring
def test_prefill_and_backward_graph_replays_match_eager(shape):
    """Summaries, route, attend and the backward captured as one HIP graph:
    every replay gives the eager outputs (forward and dq bit for bit, dk and
    dv to f32 rounding, their per-granule sums being order-free only up to
    it), with eager work and synchronizations between the replays."""
    import numpy as np
    import torch
    if shape == "qwen3":
        w = W.QWEN3_PREFILL.scaled(n_ctx=2500, kv_cap=2560, q_pos0=0, n_q=2500, planted=8)
    else:
        w = W.SMALLLM_PREFILL.scaled(batch=2, n_ctx=1500, kv_cap=1536, n_q=1500, planted=8)
    q, k, v = P.make_inputs_parallel(w)
    run = P.DeviceRun(w, q, k, v, build=False, route=False, attend=False)
    ro, cfg, dev = run.ro, run.cfg, run.q.device
    do = torch.from_numpy(W.round_to_bf16(np.random.default_rng(3).standard_normal(q.shape).astype(np.float32)))
    d_out = do.to(dev).to(run.q.dtype)
    dq = torch.empty(run.q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(run.k.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(run.k.shape, dtype=torch.float32, device=dev)
    bws = torch.empty(max(H.attend_backward_workspace_bytes(cfg, w.batch, w.q_pos0, w.n_q), 16),
                      dtype=torch.uint8, device=dev)

    def step():
        run.build()
        run.route()
        run.attend()
        H.attend_backward(cfg, run.q, w.q_pos0, run.k_rot, run.v, ro["granules"], ro["granule_count"],
                          run.out, run.lse, d_out, dq, dk, dv, bws)

    # the build writes the rows below n_ctx and the closed chunks and groups
    C, gs = w.chunk_size, w.group_size
    outs = (run.k_rot[:, :, :w.n_ctx], run.csum[:, :, :w.n_ctx // C], run.gsum[:, :, :w.n_ctx // gs],
            ro["granules"], ro["granule_count"], run.out, run.lse, dq)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    ref_kv = (dk.clone(), dv.clone())
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
        for t in outs + (dk, dv):
            t.fill_(-7) if t.dtype == torch.int32 else t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = [bool(torch.equal(a, b)) for a, b in zip(outs, ref)]
        close = [bool(torch.allclose(a, b, rtol=1e-5, atol=1e-6)) for a, b in zip((dk, dv), ref_kv)]
        print(f"[gpu] prefill graph replay {rep} ({shape}): {same} {close}", flush=True)
        assert all(same) and all(close), (rep, same, close)
        _ = (run.q.float() * 2).sum().item()  # eager work between replays
