"""GPU backward of routed exact-token attention vs the fp64 oracle
(oracle.hga_ref.attend_backward) on the GPU's own granule lists.

Tolerance: the products take bf16 operands (scaled rotated queries, keys,
values, dO, P and dS are each rounded once to 8 significant bits, relative
error <= u = 2^-8) with f32 accumulation, so each gradient element carries
an error of a few u of the magnitude of its terms.  Two bars:
* rel-L2 <= 1e-2 per tensor;
* elementwise, |gpu - oracle| <= 16 u M + 1e-6 max|M|, where M is the
  magnitude of the element's exact formula (``_magnitudes``):
  M(dv_j) = sum_i P_ij |dO_i|, M(dk~_j) = s sum_i P_ij (|dP_ij| + |D_i|) |q~_i|,
  M(dq~_i) = s sum_j P_ij (|dP_ij| + |D_i|) |k~_j|, carried through R^T as
  |cos| M_a + |sin| M_b per pair.  A CPU emulation of the kernel's roundings
  (bf16 logits' operands, P, dS and the forward output that D reads) reaches
  8.8 u on dq and 2.5 u on dk and dv (rel-L2 3e-3), so 16 u leaves a
  factor of about 2.
Keys no query sees get exactly zero.
"""
import numpy as np
import pytest

import hierarchical_kv_routing_amd as H
import workloads as W
from oracle import hga_ref as R
from tests import parity as P
from tests.random_configs import N_CONFIGS, random_workload

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
ELEM = 16 * 2.0 ** -8

CASES = {
    "qwen3_ragged": W.QWEN3_PREFILL.scaled(n_ctx=1011, kv_cap=1024, n_q=1011, planted=8),
    "qwen3_ragged_start": W.QWEN3_PREFILL.scaled(n_ctx=1011, kv_cap=1024, q_pos0=200, n_q=811, planted=8),
    "chunk_only": W.HOST_TIERED_CHUNK.scaled(n_ctx=1500, kv_cap=1536, n_q=1500, planted=8),
    "smalllm_d64": W.SMALLLM_PREFILL.scaled(batch=2, n_q_heads=4, n_kv_heads=4, n_ctx=1000,
                                            kv_cap=1024, n_q=1000, planted=8),
    "rope_wrap_p256": W.QWEN3_PREFILL.scaled(n_ctx=900, kv_cap=960, n_q=900, planted=8, rope_period=256),
    "decode_single_query": W.DECODE_64K.scaled(batch=2, n_ctx=3073, kv_cap=3136, q_pos0=3072, n_q=1),
}


def _magnitudes(w, q, k, v, gr, gc, do, units, t0):
    """M of the module docstring for dq [B,Hq,n_q,d], dk, dv [B,Hkv,kv_cap,d]
    (summed over ``units``; rows outside them stay 0)."""
    p = R.params_from_workload(w)
    G = p.Hq // p.Hkv
    sc = p.softmax_scale
    h2 = p.d // 2
    inv = R.rope_inv_freq(p.d, p.theta)

    def through_rt(m, pos):
        ang = np.multiply.outer(R.rope_position(pos, p.period), inv)
        c, s = np.abs(np.cos(ang)), np.abs(np.sin(ang))
        return np.concatenate([c * m[:, :h2] + s * m[:, h2:], s * m[:, :h2] + c * m[:, h2:]], axis=1)

    mq = np.zeros(q.shape)
    mk = np.zeros(k.shape)
    mv = np.zeros(k.shape)
    for (b, kvh, t) in units:
        gl = np.asarray(gr[b, kvh, t - t0, : int(gc[b, kvh, t - t0])], np.int64)
        tok = (gl[:, None] * p.gs + np.arange(p.gs)[None, :]).reshape(-1)
        qpos = R.unit_queries(t, w.q_pos0, w.n_q, p.C)
        qi = qpos - w.q_pos0
        mask = (tok[None, :] < t * p.C) | (tok[None, :] <= qpos[:, None])
        kk = R.rope(np.asarray(k[b, kvh][tok], np.float64), tok, p.theta, p.period)
        vv = np.asarray(v[b, kvh][tok], np.float64)
        mkk = np.zeros(kk.shape)
        for hl in range(G):
            h = kvh * G + hl
            rows = R.rope(np.asarray(q[b, h, qi], np.float64), qpos, p.theta, p.period)
            s = np.where(mask, sc * (rows @ kk.T), -np.inf)
            pr = np.exp(s - s.max(axis=1, keepdims=True))
            pr /= pr.sum(axis=1, keepdims=True)
            g = do[b, h, qi]
            dp = g @ vv.T
            dd = (g * (pr @ vv)).sum(axis=1, keepdims=True)
            a = pr * (np.abs(dp) + np.abs(dd))
            mv[b, kvh][tok] += pr.T @ np.abs(g)
            mq[b, h, qi] = through_rt(sc * (a @ np.abs(kk)), qpos)
            mkk += sc * (a.T @ np.abs(rows))
        mk[b, kvh][tok] += through_rt(mkk, tok)
    return mq, mk, mv


def _compare(name, got, ref, mag, unseen=None):
    g = got.cpu().numpy().astype(np.float64) if hasattr(got, "cpu") else np.asarray(got, np.float64)
    err = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
    bound = ELEM * mag + 1e-6 * np.abs(mag).max()
    ratio = float((np.abs(g - ref) / bound).max())
    assert err <= REL_L2 and ratio <= 1.0, (name, err, ratio)
    if unseen is not None:
        assert np.all(g[unseen] == 0), (name, "nonzero for a key no query sees")
    return round(float(err), 5), round(ratio, 4)


def _unseen_keys(w, gr, gc):
    """[B, Hkv, kv_cap, 1] mask of the keys in no unit's granule list."""
    seen = np.zeros((w.batch, w.n_kv_heads, w.kv_cap), bool)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            for u in range(gr.shape[2]):
                for gid in gr[b, h, u, : gc[b, h, u]]:
                    seen[b, h, gid * w.group_size:(gid + 1) * w.group_size] = True
    seen[:, :, w.q_pos0 + w.n_q:] = False  # past the last query: never attended
    return ~seen[..., None].repeat(w.head_dim, axis=-1)


def _check_backward(case, w, seed=0):
    """GPU backward on the GPU's own routes vs the oracle, whole tensors."""
    import torch
    q, k, v = P.make_inputs_parallel(w, seed)
    print(f"[gpu] backward {case}: {w}", flush=True)
    run = P.DeviceRun(w, q, k, v)
    dev = run.q.device
    do = W.round_to_bf16(np.random.default_rng(31).standard_normal(q.shape).astype(np.float32))
    d_out = torch.from_numpy(do).to(dev).to(torch.bfloat16)
    dq = torch.full(run.q.shape, float("nan"), dtype=torch.float32, device=dev)
    dk = torch.full(run.k.shape, float("nan"), dtype=torch.float32, device=dev)
    dv = torch.full(run.k.shape, float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(max(H.attend_backward_workspace_bytes(run.cfg, w.batch, w.q_pos0, w.n_q), 16),
                     dtype=torch.uint8, device=dev)
    ro = run.ro
    H.attend_backward(run.cfg, run.q, w.q_pos0, run.k_rot, run.v, ro["granules"], ro["granule_count"],
                      run.out, run.lse, d_out, dq, dk, dv, ws)
    torch.cuda.synchronize()
    p = R.params_from_workload(w)
    gr, gc = run.np("granules"), run.np("granule_count")
    rdq, rdk, rdv = R.attend_backward(q, w.q_pos0, w.n_q, k, v, gr, gc, do.astype(np.float64), p,
                                      t0=w.q_pos0 // w.chunk_size)
    unseen = _unseen_keys(w, gr, gc)
    mq, mk, mv = _magnitudes(w, q, k, v, gr, gc, do.astype(np.float64), P.all_units(w), w.q_pos0 // w.chunk_size)
    res = [_compare("dq", dq, rdq, mq), _compare("dk", dk, rdk, mk, unseen),
           _compare("dv", dv, rdv, mv, unseen)]
    print(f"[gpu] backward {case}: (rel_l2, max |err| / bound) dq {res[0]}, dk {res[1]}, dv {res[2]}",
          flush=True)


@pytest.mark.parametrize("case", sorted(CASES))
def test_backward_matches_oracle(case):
    _check_backward(case, CASES[case])


# The random parity shapes the backward supports (bf16, g_s a power of two
# of at least 4): chunk / group sizes, windows, budgets, GQA ratio, d,
# ragged starts and RoPE wraps beyond the named cases.
RANDOM = [i for i in range(N_CONFIGS)
          if random_workload(i).dtype == "bf16" and random_workload(i).group_size >= 4]


@pytest.mark.parametrize("i", RANDOM)
def test_backward_random_shapes(i):
    _check_backward(f"random {i}", random_workload(i), seed=i)


def test_backward_deterministic_except_atomics():
    """dq has no atomics: bitwise repeatable; dk and dv are sums of atomic
    adds and agree to f32 rounding between two calls."""
    import torch
    w = CASES["qwen3_ragged"]
    q, k, v = P.make_inputs_parallel(w)
    run = P.DeviceRun(w, q, k, v)
    dev = run.q.device
    d_out = torch.from_numpy(W.round_to_bf16(np.random.default_rng(32).standard_normal(q.shape).astype(np.float32))
                             ).to(dev).to(torch.bfloat16)
    ws = torch.empty(max(H.attend_backward_workspace_bytes(run.cfg, w.batch, w.q_pos0, w.n_q), 16),
                     dtype=torch.uint8, device=dev)
    outs = []
    for _ in range(2):
        dq = torch.empty(run.q.shape, dtype=torch.float32, device=dev)
        dk = torch.empty(run.k.shape, dtype=torch.float32, device=dev)
        dv = torch.empty(run.k.shape, dtype=torch.float32, device=dev)
        H.attend_backward(run.cfg, run.q, w.q_pos0, run.k_rot, run.v, run.ro["granules"],
                          run.ro["granule_count"], run.out, run.lse, d_out, dq, dk, dv, ws)
        outs.append((dq, dk, dv))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0])
    for i in (1, 2):
        a, b = outs[0][i], outs[1][i]
        assert torch.allclose(a, b, rtol=1e-5, atol=1e-6 * float(a.abs().max()))


def test_backward_qwen3_32k_sampled():
    """The full Qwen3-shaped prefill (n = 32768, the configuration bench.py
    times): dq of sampled units, and dk, dv of the tokens of sampled granules
    together with every unit that lists them (so their sums are complete),
    against the oracle on the GPU's own granule lists.  Sink granules (listed
    by every unit of the slab) are left out for the oracle's time."""
    import torch
    w = W.QWEN3_PREFILL
    q, k, v = P.make_inputs_parallel(w)
    print("[gpu] backward qwen3 32k: inputs ready", flush=True)
    run = P.DeviceRun(w, q, k, v)
    dev = run.q.device
    do = W.round_to_bf16(np.random.default_rng(41).standard_normal(q.shape).astype(np.float32))
    d_out = torch.from_numpy(do).to(dev).to(torch.bfloat16)
    dq = torch.empty(run.q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(run.k.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(run.k.shape, dtype=torch.float32, device=dev)
    ws = torch.empty(max(H.attend_backward_workspace_bytes(run.cfg, w.batch, w.q_pos0, w.n_q), 16),
                     dtype=torch.uint8, device=dev)
    H.attend_backward(run.cfg, run.q, w.q_pos0, run.k_rot, run.v, run.ro["granules"], run.ro["granule_count"],
                      run.out, run.lse, d_out, dq, dk, dv, ws)
    torch.cuda.synchronize()
    print("[gpu] backward qwen3 32k: gpu done", flush=True)
    gr, gc = run.np("granules"), run.np("granule_count")
    nqc = gr.shape[2]
    sink = w.n_sink_chunks * (w.chunk_size // w.group_size)
    rng = np.random.default_rng(42)
    units, picks = set(), []
    for (b, h) in [(0, 0), (0, 3)]:
        holders = {}
        for t in range(nqc):
            for g in gr[b, h, t, : gc[b, h, t]].tolist():
                holders.setdefault(g, []).append(t)
        cand = sorted(g for g, ts in holders.items() if g >= sink and 2 <= len(ts) <= 16)
        for g in rng.choice(cand, 3, replace=False).tolist():
            picks.append((b, h, g))
            units.update((b, h, t) for t in holders[g])
    units.update([(0, 1, 7), (0, 2, 300)])
    units = sorted(units)
    p = R.params_from_workload(w)
    rdq, rdk, rdv = R.attend_backward(q, w.q_pos0, w.n_q, k, v, gr, gc, do.astype(np.float64), p,
                                      t0=0, units=units)
    mq, mk, mv = _magnitudes(w, q, k, v, gr, gc, do.astype(np.float64), units, 0)
    G = w.n_q_heads // w.n_kv_heads
    C = w.chunk_size
    gs = w.group_size
    qsel = [(b, h * G + hl, t * C + i) for (b, h, t) in units for hl in range(G) for i in range(C)]
    bi, hi, qi = (torch.tensor([s[j] for s in qsel], device=dev) for j in range(3))
    got_q = dq[bi, hi, qi].cpu().numpy().astype(np.float64)
    want_q = rdq[np.array([s[0] for s in qsel]), np.array([s[1] for s in qsel]), np.array([s[2] for s in qsel])]
    tsel = [(b, h, g * gs + j) for (b, h, g) in picks for j in range(gs)]
    tb, th, tt = (torch.tensor([s[j] for s in tsel], device=dev) for j in range(3))
    ib, ih, it = (np.array([s[j] for s in tsel]) for j in range(3))
    qb, qh, qq = (np.array([s[j] for s in qsel]) for j in range(3))
    res = []
    for name, got, want, mag in (("dq", got_q, want_q, mq[qb, qh, qq]),
                                 ("dk", dk[tb, th, tt].cpu().numpy().astype(np.float64), rdk[ib, ih, it],
                                  mk[ib, ih, it]),
                                 ("dv", dv[tb, th, tt].cpu().numpy().astype(np.float64), rdv[ib, ih, it],
                                  mv[ib, ih, it])):
        res.append((name,) + _compare(name, got, want, mag))
    print(f"[gpu] backward qwen3 32k: {len(units)} units, {len(picks)} granules: {res}", flush=True)
