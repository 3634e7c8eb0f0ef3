"""Shared GPU-vs-oracle parity helpers (imported by the gpu tests).

Tolerances (written here, used by every parity test):

* Summaries and the f32 rotated key cache: |gpu - oracle| <= 2e-5 absolute.
  The GPU forms each RoPE angle in double, reduces it to [-pi, pi] and
  evaluates an f32 sincos: about 2.5e-7 rad of error, i.e. <= 4e-6 on a
  rotated element of magnitude <= 15; f32 sums of 64 such terms add <= 1e-6.
* bf16 rotated key cache: one bf16 rounding, <= 2^-8 |x| + 2e-5.
* Routing: chunk / group index lists bit-exact, except units whose oracle
  top-K margin s_(K) - s_(K+1) is positive and below 1e-3 |s_(K)| (near-ties,
  counted and reported); there every GPU-selected id must still score within
  that band of the oracle's K-th score.  An exact tie (margin 0) is no
  exception: the lowest index wins.  Granule lists bit-exact given the
  selections.
* Attention, computed by the oracle on the GPU's own granule lists.
  f32: max-abs <= 1e-5 and rel-L2 <= 1e-5 against exact keys; LSE <= 1e-5.
  bf16, three checks on every compared row:
  (a) against exact float64 rotated keys (the plain definition): rel-L2 <=
      1e-2, and every output element and every LSE within the rounding
      bound derived from the bf16 arithmetic (``_rounding_bound``: bf16
      rounding of the scaled rotated query and of the rotated keys moves a
      logit by at most 2u scale sum_d |q~_d k~_d|, u = 2^-8; P and the output
      are rounded to bf16 once more);
  (b) against the rotated keys as a bf16 key cache holds them (each rotated
      key rounded to bf16, the reading a bf16 model's post-RoPE key cache
      gives): max-abs <= 2e-2 and rel-L2 <= 1e-2;
  (c) recorded, not asserted: max-abs against exact keys and the number of
      rows whose max-abs against exact keys exceeds 2e-2 (a row whose two
      largest logits compete loses up to ~3e-2 to the key rounding alone).
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
    slabs = sorted({(b, h) for (b, h, _) in units})
    with ThreadPoolExecutor(max_workers=16) as ex:
        done = ex.map(lambda bh: R.summaries(k[bh[0], bh[1]].astype(np.float64), n_sum, p), slabs)
        sums = dict(zip(slabs, done))
    B, Hkv = w.batch, w.n_kv_heads
    nc = sums[next(iter(sums))][0].shape[0]
    ng = sums[next(iter(sums))][1].shape[0]
    cs = np.zeros((B, Hkv, nc, p.d))
    gs = np.zeros((B, Hkv, ng, p.d))
    for (b, h), (c, g) in sums.items():
        cs[b, h], gs[b, h] = c, g
    return R.route(q, w.q_pos0, w.n_q, cs, gs, p, units=units)


def compare_routes(run: DeviceRun, orc: dict, units, name=None):
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
            # an exact tie (margin 0) has one answer: the lowest index
            assert 0 < info["margin_c"] < band, ((b, h, t), g_ch, info["sel_chunks"], info["margin_c"])
            sc = dict(zip(info["mid"], info["chunk_scores"]))
            assert all(sc[m] >= info["s_kc"] - band for m in g_ch), (b, h, t)
            near += 1
            continue
        if p.Kg > 0 and g_gr != info["sel_groups"]:
            band = TIE_REL * abs(info["s_kg"])
            assert 0 < info["margin_g"] < band, ((b, h, t), g_gr, info["sel_groups"], info["margin_g"])
            sg = dict(zip(info["group_cands"], info["group_scores"]))
            assert all(sg[x] >= info["s_kg"] - band for x in g_gr), (b, h, t)
            near += 1
            continue
        exact += 1
    ties = sum(1 for u in units if orc["info"][u]["margin_c"] == 0 or orc["info"][u]["margin_g"] == 0)
    record("routes", name or w.name, units=len(units), exact=exact, near_tie=near, exact_ties=ties)
    return exact, near


class AttnStats(tuple):
    """(max_abs, rel_l2, lse_err) against exact float64 keys, plus the
    detail of the comparison as attributes."""

    def __new__(cls, **kw):
        obj = super().__new__(cls, (kw["max_abs"], kw["rel_l2"], kw["lse_err"]))
        obj.__dict__.update(kw)
        return obj

    def as_dict(self):
        return dict(self.__dict__)


# Results of every attention comparison made in this process (reported by
# conftest.py at the end of a run and written to gpurun_out/ when present).
RECORDS = []


def record(kind, name, **kw):
    RECORDS.append(dict(kind=kind, name=name, **kw))


def _rounding_bound(w, p, rows, kk, vv, mask, o, lse):
    """Per-element bound on |gpu - exact| for bf16 attention of query rows
    ``rows`` [R,d] (rotated, float64) over keys kk [nk,d] (rotated, exact),
    values vv, with the exact output o [R,d] and log-sum-exp lse [R].

    The bf16 path rounds scale*q~ and k~ to bf16 (relative error <= u = 2^-8
    each) and accumulates in f32, so logit j of a row moves by at most
      E_j = scale * sum_d |q~_d k~_jd| * (2u + u^2 + 2^-16)
    (the last term covers the f32 sums over d <= 128 and the f32 RoPE).  With
    E-bar = log sum_j p_j e^{E_j}, softmax weights move to p'_j with
    |p'_j - p_j| <= p_j (e^{E_j + E-bar} - 1), and since sum_j (p'_j - p_j) = 0,
      |o'_d - o_d| <= sum_j p_j (e^{E_j+E-bar} - 1) |v_jd - o_d|
                   <= sum_j p_j (e^{E_j+E-bar} - 1) (|v_jd| + |o_d|).
    P is rounded to bf16 for the PV product (<= u sum_j p'_j |v_jd|) and the
    output to bf16 (<= u |o'_d|).  The LSE moves by at most E-bar, plus f32
    rounding of its sum over nk terms (nk 2^-24) and of the log.
    Returns (bound_out [R,d], bound_lse [R])."""
    u = 2.0 ** -8
    scale = p.softmax_scale
    E = scale * (np.abs(rows) @ np.abs(kk).T) * (2 * u + u * u + 2.0 ** -16)
    E = np.where(mask, E, 0.0)
    logits = scale * (rows @ kk.T)
    pr = np.where(mask, np.exp(np.where(mask, logits, -np.inf) - lse[:, None]), 0.0)
    ebar = np.log(np.sum(pr * np.exp(E), axis=1))
    grow = np.exp(E + ebar[:, None])
    av = np.abs(vv)
    ao = np.abs(o)
    w1 = pr * (grow - 1.0)
    t1 = w1 @ av + w1.sum(axis=1)[:, None] * ao
    t2 = u * ((pr * grow) @ av)
    t3 = u * (ao + t1 + t2)
    b_out = 1.02 * (t1 + t2 + t3) + 2e-5
    nk = mask.sum(axis=1)
    b_lse = 1.02 * ebar + (nk + 8) * 2.0 ** -24 + 2.0 ** -22 * np.abs(lse) + 2e-6
    return b_out, b_lse


def _unit_bounds(w, p, q, k, v, tok, qpos, mask, b, kvh, o_ref, l_ref, bo, bl):
    """Fill bo / bl (like o_ref / l_ref) for the rows of one unit."""
    G = p.Hq // p.Hkv
    kk = R.rope(np.asarray(k[b, kvh][tok], np.float64), tok, p.theta, p.period)
    vv = np.asarray(v[b, kvh][tok], np.float64)
    qi = qpos - w.q_pos0
    for hl in range(G):
        h = kvh * G + hl
        rows = R.rope(np.asarray(q[b, h, qi, :], np.float64), qpos, p.theta, p.period)
        o_b, l_b = _rounding_bound(w, p, rows, kk, vv, mask, o_ref[b, h, qi], l_ref[b, h, qi])
        bo[b, h, qi] = o_b
        bl[b, h, qi] = l_b


def _compare(w, name, out, lse, o_ref, l_ref, o_cached=None, l_cached=None, bo=None, bl=None):
    """The acceptance rule for attention outputs (see the module docstring)."""
    sel = ~np.isnan(o_ref)
    assert sel.any()
    diff = np.abs(out - o_ref)
    max_abs = float(diff[sel].max())
    rel_l2 = float(np.linalg.norm((out - o_ref)[sel]) / max(np.linalg.norm(o_ref[sel]), 1e-30))
    lsel = ~np.isnan(l_ref)
    lerr = np.abs(lse - l_ref)
    lse_err = float(lerr[lsel].max())
    tol_abs, tol_rel = TOL[w.dtype]
    rowmax = np.where(sel, diff, 0.0).max(axis=-1)
    rows = int(np.count_nonzero(lsel))
    rows_over = int(np.count_nonzero(rowmax[lsel] > tol_abs))
    kw = dict(dtype=w.dtype, rows=rows, max_abs=max_abs, rel_l2=rel_l2, lse_err=lse_err,
              rows_over_abs_tol=rows_over)
    if w.dtype != "bf16":
        record("attention", name, **kw)
        assert max_abs <= tol_abs and rel_l2 <= tol_rel, (name, max_abs, rel_l2)
        assert lse_err <= tol_abs, (name, lse_err)
        return AttnStats(**kw)
    # against the rotated keys held in bf16 (the stated cache reading): the full bar
    dc = np.abs(out - o_cached)[sel]
    kw["max_abs_cached_keys"] = float(dc.max())
    kw["rel_l2_cached_keys"] = float(np.linalg.norm((out - o_cached)[sel])
                                     / max(np.linalg.norm(o_cached[sel]), 1e-30))
    # against exact keys: every element and every LSE within its rounding bound
    ratio = float((diff[sel] / bo[sel]).max())
    lratio = float((lerr[lsel] / bl[lsel]).max())
    kw.update(bound_ratio_max=ratio, lse_bound_ratio_max=lratio)
    record("attention", name, **kw)
    assert kw["max_abs_cached_keys"] <= tol_abs and kw["rel_l2_cached_keys"] <= tol_rel, (name, kw)
    assert rel_l2 <= tol_rel, (name, "rel-L2 against exact keys", kw)
    assert ratio <= 1.0, (name, "output beyond its rounding bound", kw)
    assert lratio <= 1.0, (name, "LSE beyond its rounding bound", kw)
    return AttnStats(**kw)


def check_attention(run: DeviceRun, q, k, v, units, out=None, lse=None, name=None):
    """GPU attention of ``units`` against the oracle on the GPU's own granule
    lists (the acceptance rule is in the module docstring)."""
    import dataclasses
    w = run.w
    p = R.params_from_workload(w)
    gr, gc = run.np("granules"), run.np("granule_count")
    t0 = w.q_pos0 // w.chunk_size
    o_ref, l_ref = R.attend_given(q, w.q_pos0, w.n_q, k, v, gr, gc, p, t0=t0, units=units)
    out = run.np("out") if out is None else out
    lse = run.np("lse") if lse is None else lse
    o_c = l_c = bo = bl = None
    if w.dtype == "bf16":
        o_c, l_c = R.attend_given(q, w.q_pos0, w.n_q, k, v, gr, gc,
                                  dataclasses.replace(p, key_cache="bf16"), t0=t0, units=units)
        bo = np.full(o_ref.shape, np.nan)
        bl = np.full(l_ref.shape, np.nan)
        for (b, kvh, t) in units:
            gl = np.asarray(gr[b, kvh, t - t0, : int(gc[b, kvh, t - t0])], np.int64)
            tok = (gl[:, None] * p.gs + np.arange(p.gs)[None, :]).reshape(-1)
            qpos = R.unit_queries(t, w.q_pos0, w.n_q, p.C)
            mask = (tok[None, :] < t * p.C) | (tok[None, :] <= qpos[:, None])
            _unit_bounds(w, p, q, k, v, tok, qpos, mask, b, kvh, o_ref, l_ref, bo, bl)
    return _compare(w, name or w.name, out, lse, o_ref, l_ref, o_c, l_c, bo, bl)


def check_dense(w, out, lse, q, k, v, heads=None, q_index=None, name=None):
    """GPU dense causal attention (Eq. 1) against the oracle's, on the rows
    of ``heads`` x ``q_index`` (all when None); same acceptance rule."""
    import dataclasses
    p = R.params_from_workload(w)
    o_ref, l_ref = R.dense_causal(q, w.q_pos0, w.n_q, k, v, p, heads=heads, q_index=q_index)
    o_c = l_c = bo = bl = None
    if w.dtype == "bf16":
        o_c, l_c = R.dense_causal(q, w.q_pos0, w.n_q, k, v, dataclasses.replace(p, key_cache="bf16"),
                                  heads=heads, q_index=q_index)
        bo = np.full(o_ref.shape, np.nan)
        bl = np.full(l_ref.shape, np.nan)
        qi = np.arange(w.n_q) if q_index is None else np.asarray(q_index)
        qpos = w.q_pos0 + qi
        nk = int(qpos.max()) + 1
        tok = np.arange(nk)
        mask = tok[None, :] <= qpos[:, None]
        G = p.Hq // p.Hkv
        for b in range(w.batch):
            for kvh in range(p.Hkv):
                if heads is not None and not any(h // G == kvh for h in heads):
                    continue
                _unit_bounds(w, p, q, k, v, tok, qpos, mask, b, kvh, o_ref, l_ref, bo, bl)
        if heads is not None:
            keep = np.zeros(p.Hq, bool)
            keep[list(heads)] = True
            bo[:, ~keep] = np.nan
            bl[:, ~keep] = np.nan
    return _compare(w, name or (w.name + ":dense"), out, lse, o_ref, l_ref, o_c, l_c, bo, bl)


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
