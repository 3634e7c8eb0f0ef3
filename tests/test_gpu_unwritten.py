"""Keys after a call's last query are never read into a result.  The rotated
K and V there may be memory the caller has not written yet (a decode cache
filled up to the current token); here it is set to NaN, and attention (bf16,
f32 and the decode form) and the backward must return exactly what they
return with finite values there.  P of such a key is zero, but a product of
a zero P with a NaN V would still be NaN."""
import numpy as np
import pytest

import hierarchical_kv_routing_amd as H
import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_prefill": W.QWEN3_PREFILL.scaled(n_ctx=1011, kv_cap=1088, n_q=1011, planted=8),
    "bf16_ragged_start": W.QWEN3_PREFILL.scaled(n_ctx=1011, kv_cap=1088, q_pos0=200, n_q=811, planted=8),
    "f32": W.TINY_F32.scaled(n_ctx=1000, kv_cap=1088, n_q=1000),
    "decode": W.DECODE_64K.scaled(batch=2, n_ctx=3073, kv_cap=3136, q_pos0=3072, n_q=1),
}


def _poisoned(run, w):
    """Copies of k_rot and v with NaN from the first position after the last query."""
    end = w.q_pos0 + w.n_q
    assert end < w.kv_cap
    k_rot, v = run.k_rot.clone(), run.v.clone()
    k_rot[:, :, end:] = float("nan")
    v[:, :, end:] = float("nan")
    return k_rot, v


@pytest.mark.parametrize("case", sorted(CASES))
def test_attend_ignores_memory_after_last_query(case):
    import torch
    w = CASES[case]
    q, k, v = P.make_inputs_parallel(w)
    print(f"[gpu] unwritten tail, attend {case}: {w}", flush=True)
    run = P.DeviceRun(w, q, k, v)
    k_rot, vv = _poisoned(run, w)
    out = torch.full_like(run.out, float("nan"))
    lse = torch.full_like(run.lse, float("nan"))
    H.attend(run.cfg, run.q, w.q_pos0, k_rot, vv, run.ro["granules"], run.ro["granule_count"],
             out, lse, run.aws)
    torch.cuda.synchronize()
    assert torch.equal(out, run.out) and torch.equal(lse, run.lse)


def test_backward_ignores_memory_after_last_query():
    import torch
    w = CASES["bf16_prefill"]
    q, k, v = P.make_inputs_parallel(w)
    print(f"[gpu] unwritten tail, backward: {w}", flush=True)
    run = P.DeviceRun(w, q, k, v)
    dev = run.q.device
    do = W.round_to_bf16(np.random.default_rng(33).standard_normal(q.shape).astype(np.float32))
    d_out = torch.from_numpy(do).to(dev).to(torch.bfloat16)
    ws = torch.empty(max(H.attend_backward_workspace_bytes(run.cfg, w.batch, w.q_pos0, w.n_q), 16),
                     dtype=torch.uint8, device=dev)
    res = []
    for k_rot, vv in ((run.k_rot, run.v), _poisoned(run, w)):
        dq = torch.full(run.q.shape, float("nan"), dtype=torch.float32, device=dev)
        dk = torch.full(run.k.shape, float("nan"), dtype=torch.float32, device=dev)
        dv = torch.full(run.k.shape, float("nan"), dtype=torch.float32, device=dev)
        H.attend_backward(run.cfg, run.q, w.q_pos0, k_rot, vv, run.ro["granules"], run.ro["granule_count"],
                          run.out, run.lse, d_out, dq, dk, dv, ws)
        res.append((dq, dk, dv))
    torch.cuda.synchronize()
    (dq0, dk0, dv0), (dq1, dk1, dv1) = res
    assert torch.equal(dq0, dq1)
    end = w.q_pos0 + w.n_q
    for a, b in ((dk0, dk1), (dv0, dv1)):
        assert bool(torch.isfinite(b).all())
        assert torch.allclose(a, b, rtol=1e-5, atol=1e-6 * float(a.abs().max()))
        assert bool((b[:, :, end:] == 0).all())
