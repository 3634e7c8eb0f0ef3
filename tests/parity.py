"""Shared GPU-vs-oracle parity helpers (imported by the gpu tests).

Tolerances (written here, used by every parity test):

* Summaries and the f32 rotated key cache: |gpu - oracle| <= 2e-5 absolute.
  The GPU forms each RoPE angle in double, reduces it to [-pi, pi] and
  evaluates an f32 sincos: about 2.5e-7 rad of error, i.e. <= 4e-6 on a
  rotated element of magnitude <= 15; f32 sums of 64 such terms add <= 1e-6.
* bf16 rotated key cache: one bf16 rounding, <= 2^-8 |x| + 2e-5.
* Routing: chunk / group index lists bit-exact, except units whose oracle
  top-K margin s_(K) - s_(K+1) is below 1e-3 |s_(K)| (near-ties, counted and
  reported); there every GPU-selected id must still score within that band of
  the oracle's K-th score.  Granule lists bit-exact given the selections.
* Attention, computed by the oracle on the GPU's own granule lists:
  bf16 max-abs <= 2e-2 and rel-L2 <= 1e-2; f32 max-abs <= 1e-5 and rel-L2 <= 1e-5.
* Log-sum-exp: the bf16 path rounds the scaled rotated query and the rotated
  keys to bf16, so each product q_i k_i carries a relative error below 2^-8
  and every logit moves by at most 2^-8 * scale * sum_i |q_i k_i| <=
  2^-8 * scale * |q| * |k|; the LSE moves by at most the largest logit move:
  tol(row) = 2^-8 * scale * |q_row| * max_j |k_j| + 1e-5.  f32: 1e-5.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import hierarchical_kv_routing_amd as H
import workloads as W
from oracle import hga_ref as R

SUM_ATOL = 2e-5
TIE_REL = 1e-3
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-5, 1e-5)}


def torch_dtype(w):
    import torch
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def make_inputs_parallel(w, seed=0, threads=16):
    """workloads.make_inputs with slabs drawn on a thread pool."""
    return W.make_inputs(w, seed, threads=threads)


class DeviceRun:
    """Device tensors and outputs of one pass of the whole path."""

    def __init__(self, w, q, k, v, cfg=None, build=True, route=True, attend=True):
        import torch
        self.w = w
        self.cfg = cfg or H.Config.from_workload(w)
        dev = torch.device("cuda:0")
        dt = torch_dtype(w)
        self.q = torch.from_numpy(q).to(dev).to(dt)
        self.k = torch.from_numpy(k).to(dev).to(dt)
        self.v = torch.from_numpy(v).to(dev).to(dt)
        B, Hkv, cap, d = self.k.shape
        c = self.cfg
        self.k_rot = torch.zeros_like(self.k)
        self.csum = torch.zeros((B, Hkv, cap // c.chunk_size, d), dtype=torch.float32, device=dev)
        self.gsum = torch.zeros((B, Hkv, cap // c.group_size, d), dtype=torch.float32, device=dev)
        self.ro = H.route_outputs(c, B, w.q_pos0, w.n_q, dev)
        self.out = torch.zeros_like(self.q)
        self.lse = torch.zeros(self.q.shape[:3], dtype=torch.float32, device=dev)
        aw = H.attend_workspace_bytes(c, B, w.q_pos0, w.n_q)
        self.aws = torch.empty(max(aw, 16), dtype=torch.uint8, device=dev)
        if build:
            self.build()
        if route:
            self.route()
        if attend:
            self.attend()
        torch.cuda.synchronize()

    def build(self):
        H.build_summaries(self.cfg, self.k, 0, self.w.n_ctx, self.k_rot, self.csum, self.gsum)

    def route(self):
        r = self.ro
        H.route(self.cfg, self.q, self.w.q_pos0, self.csum, self.gsum, self.k.shape[2],
                r["chunk_idx"], r["group_idx"], r["granules"], r["granule_count"], r["workspace"])

    def attend(self):
        r = self.ro
        H.attend(self.cfg, self.q, self.w.q_pos0, self.k_rot, self.v, r["granules"],
                 r["granule_count"], self.out, self.lse, self.aws)

    def np(self, name):
        import torch
        t = getattr(self, name) if hasattr(self, name) else self.ro[name]
        return t.float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float32) else t.cpu().numpy()


def check_summaries(run: DeviceRun, k, slabs=None):
    """GPU summaries and rotated keys vs the oracle on the listed (b, kvh) slabs."""
    w = run.w
    p = R.params_from_workload(w)
    csum, gsum, krot = run.np("csum"), run.np("gsum"), run.np("k_rot")
    if slabs is None:
        slabs = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    n = w.n_ctx
    worst = 0.0
    for (b, h) in slabs:
        kk = k[b, h].astype(np.float64)
        oc, og = R.summaries(kk, n, p)
        dc = np.abs(csum[b, h, : oc.shape[0]] - oc).max(initial=0.0)
        dg = np.abs(gsum[b, h, : og.shape[0]] - og).max(initial=0.0)
        assert dc <= SUM_ATOL and dg <= SUM_ATOL, (b, h, dc, dg)
        ref = R.rope(kk[:n], np.arange(n), p.theta, p.period)
        err = np.abs(krot[b, h, :n] - ref)
        if w.dtype == "bf16":
            assert np.all(err <= 2.0 ** -8 * np.abs(ref) + SUM_ATOL), (b, h, err.max())
        else:
            assert err.max(initial=0.0) <= SUM_ATOL, (b, h, err.max())
        worst = max(worst, dc, dg)
    return worst


def oracle_route(run: DeviceRun, q, k, units):
    """Oracle routing (own f64 summaries) of the given units."""
    w = run.w
    p = R.params_from_workload(w)
    n_sum = w.n_ctx
    sums = {}
    for (b, h, _) in units:
        if (b, h) not in sums:
            sums[(b, h)] = R.summaries(k[b, h].astype(np.float64), n_sum, p)
    B, Hkv = w.batch, w.n_kv_heads
    nc = sums[next(iter(sums))][0].shape[0]
    ng = sums[next(iter(sums))][1].shape[0]
    cs = np.zeros((B, Hkv, nc, p.d))
    gs = np.zeros((B, Hkv, ng, p.d))
    for (b, h), (c, g) in sums.items():
        cs[b, h], gs[b, h] = c, g
    return R.route(q, w.q_pos0, w.n_q, cs, gs, p, units=units)


def compare_routes(run: DeviceRun, orc: dict, units):
    """Returns (exact, near_tie) counts; asserts every other unit matches."""
    w = run.w
    p = R.params_from_workload(w)
    ci, gi = run.np("chunk_idx"), run.np("group_idx")
    gr, gc = run.np("granules"), run.np("granule_count")
    t0 = w.q_pos0 // w.chunk_size
    exact = near = 0
    for (b, h, t) in units:
        info = orc["info"][(b, h, t)]
        u = t - t0
        g_ch = [int(x) for x in ci[b, h, u] if x >= 0] if p.Kc > 0 else []
        g_gr = [int(x) for x in gi[b, h, u] if x >= 0] if p.Kg > 0 else []
        qlast = min((t + 1) * p.C, w.q_pos0 + w.n_q) - 1
        # the granule list is exact given the GPU's own selections
        want = R.visible_granules(t, qlast, g_ch, g_gr, p)
        got = [int(x) for x in gr[b, h, u, : gc[b, h, u]]]
        assert got == want, ((b, h, t), got, want)
        assert all(x == -1 for x in gr[b, h, u, gc[b, h, u]:])
        if g_ch != info["sel_chunks"]:
            band = TIE_REL * abs(info["s_kc"])
            assert info["margin_c"] < band, ((b, h, t), g_ch, info["sel_chunks"], info["margin_c"])
            sc = dict(zip(info["mid"], info["chunk_scores"]))
            assert all(sc[m] >= info["s_kc"] - band for m in g_ch), (b, h, t)
            near += 1
            continue
        if p.Kg > 0 and g_gr != info["sel_groups"]:
            band = TIE_REL * abs(info["s_kg"])
            assert info["margin_g"] < band, ((b, h, t), g_gr, info["sel_groups"], info["margin_g"])
            sg = dict(zip(info["group_cands"], info["group_scores"]))
            assert all(sg[x] >= info["s_kg"] - band for x in g_gr), (b, h, t)
            near += 1
            continue
        exact += 1
    return exact, near


def check_attention(run: DeviceRun, q, k, v, units, out=None, lse=None):
    """Oracle attention on the GPU's granule lists for ``units``: within the
    tolerances against the keys as the workload's dtype caches them, and
    (bf16) within the rel-L2 bar against exact float64 keys too."""
    w = run.w
    p = R.params_from_workload(w)
    gr, gc = run.np("granules"), run.np("granule_count")
    o_ref, l_ref = R.attend_given(q, w.q_pos0, w.n_q, k, v, gr, gc, p,
                                  t0=w.q_pos0 // w.chunk_size, units=units)
    out = run.np("out") if out is None else out
    lse = run.np("lse") if lse is None else lse
    res = compare_out(w, out, lse, o_ref, l_ref, q=q, k=k)
    if w.dtype == "bf16":
        import dataclasses
        o_x, _ = R.attend_given(q, w.q_pos0, w.n_q, k, v, gr, gc,
                                dataclasses.replace(p, key_cache="f64"),
                                t0=w.q_pos0 // w.chunk_size, units=units)
        sel = ~np.isnan(o_x)
        rel = float(np.linalg.norm(out[sel] - o_x[sel]) / max(np.linalg.norm(o_x[sel]), 1e-30))
        assert rel <= TOL["bf16"][1], ("rel-L2 against exact keys", rel)
    return res


def lse_tolerance(w, q, k):
    """Per-row LSE bound [B,Hq,n_q] (see the module docstring)."""
    if w.dtype != "bf16":
        return np.full(q.shape[:3], 1e-5)
    scale = 1.0 / math.sqrt(w.head_dim)
    qn = np.linalg.norm(q.astype(np.float64), axis=-1)                    # [B,Hq,n_q]
    kmax = np.linalg.norm(k[:, :, : w.n_ctx].astype(np.float64), axis=-1).max(axis=-1)  # [B,Hkv]
    kmax = np.repeat(kmax, w.group_ratio, axis=1)[:, :, None]
    return 2.0 ** -8 * scale * qn * kmax + 1e-5


def compare_out(w, out, lse, o_ref, l_ref, q=None, k=None):
    sel = ~np.isnan(o_ref)
    assert sel.any()
    diff = np.abs(out[sel] - o_ref[sel])
    max_abs = float(diff.max())
    rel_l2 = float(np.linalg.norm(out[sel] - o_ref[sel]) / max(np.linalg.norm(o_ref[sel]), 1e-30))
    lsel = ~np.isnan(l_ref)
    lerr = np.abs(lse[lsel] - l_ref[lsel])
    tol_abs, tol_rel = TOL[w.dtype]
    assert max_abs <= tol_abs and rel_l2 <= tol_rel, (max_abs, rel_l2)
    if q is not None:
        ltol = lse_tolerance(w, q, k)[lsel]
        assert np.all(lerr <= ltol), float((lerr / ltol).max())
    else:
        assert lerr.max() <= tol_abs, float(lerr.max())
    return max_abs, rel_l2, float(lerr.max())


def all_units(w):
    t0 = w.q_pos0 // w.chunk_size
    t1 = (w.q_pos0 + w.n_q - 1) // w.chunk_size
    return [(b, h, t) for b in range(w.batch) for h in range(w.n_kv_heads) for t in range(t0, t1 + 1)]


def sample_units(w, n, seed=0):
    """Deterministic sample: always the last query chunk of the first and
    last slabs, plus random units."""
    units = all_units(w)
    rng = np.random.default_rng(seed)
    last = max(u[2] for u in units)
    pick = {(0, 0, last), (w.batch - 1, w.n_kv_heads - 1, last)}
    while len(pick) < min(n, len(units)):
        pick.add(units[int(rng.integers(len(units)))])
    return sorted(pick)
