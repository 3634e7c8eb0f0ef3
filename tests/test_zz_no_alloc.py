"""hga_attend_noalloc (the entry point for callers that cannot allocate)
against hga_attend on the same inputs: two calls in a row on one device, the
second with a smaller input, so the second runs on the static scratch the
first left behind.  Both decode-shaped calls split each unit's keys over
several workgroups, whose partials are what the scratch holds; outputs and
LSE must equal hga_attend's bit for bit (same kernels and plan)."""
import pytest

import hierarchical_kv_routing_amd as H
import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu

CALLS = [
    W.DECODE_64K.scaled(batch=4, n_ctx=20481, kv_cap=20544, q_pos0=20480),
    W.DECODE_64K.scaled(batch=2, n_ctx=8193, kv_cap=8256, q_pos0=8192),
]


def test_attend_noalloc_matches_attend_two_calls():
    import torch
    for i, w in enumerate(CALLS):
        print(f"[gpu] noalloc call {i}: {w}", flush=True)
        cfg = H.Config.from_workload(w)
        need = H.attend_workspace_bytes(cfg, w.batch, w.q_pos0, w.n_q)
        assert 0 < need <= H.attend_noalloc_max_scratch_bytes()
        q, k, v = P.make_inputs_parallel(w, seed=60 + i)
        run = P.DeviceRun(w, q, k, v)
        out = torch.full_like(run.out, float("nan"))
        lse = torch.full_like(run.lse, float("nan"))
        H.attend_noalloc(run.cfg, run.q, w.q_pos0, run.k_rot, run.v, run.ro["granules"],
                         run.ro["granule_count"], out, lse)
        torch.cuda.synchronize()
        same = bool(torch.equal(out, run.out)) and bool(torch.equal(lse, run.lse))
        assert same, (i, float((out.float() - run.out.float()).abs().max()))
