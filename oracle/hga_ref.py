"""Vectorised float64 oracle of HGA routed exact-token attention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Every array is
float64; inputs are widened exactly from the float32 / bfloat16 values the
generators produce, and every step is exact float64 arithmetic by default.
One rounding can be modelled on request, as a stated reading of a point the
pages leave open: ``Params.key_cache`` = "bf16" / "f32" holds the rotated
keys the attention reads in that dtype (``round_to_cache``), as a model of
that dtype caches its post-RoPE keys.  The default, "f64", is the plain
definition (exact rotated keys).

Layouts: q [B][Hq][n_q][d] (query qi sits at position q_pos0 + qi);
k, v [B][Hkv][kv_cap][d] (slot j holds position j); chunk summaries
[B][Hkv][n_closed_chunks][d]; group summaries [B][Hkv][n_closed_groups][d].
A granule is one g_s-token block; granule g covers tokens [g*g_s, (g+1)*g_s).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Params:
    C: int            # chunk size
    gs: int           # group size g_s, C % gs == 0
    F: int            # always-visible first (sink) chunks
    L: int            # always-visible recent closed chunks
    Kc: int           # routed chunks
    Kg: int           # routed groups; 0 = routed chunks are opened whole
    n_hf: int         # pairs [0, n_hf) are high frequency
    theta: float      # RoPE base
    Hq: int
    Hkv: int
    d: int
    scale: float = 0.0  # 0 -> 1/sqrt(d)
    period: int = 0     # RoPE positions wrap modulo period; 0 = absolute
    key_cache: str = "f64"  # rotated keys as attention reads them: exact ("f64"), or held in "bf16" / "f32"

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale else 1.0 / math.sqrt(self.d)

    @property
    def groups_per_chunk(self) -> int:
        return self.C // self.gs


def params_from_workload(w) -> Params:
    return Params(C=w.chunk_size, gs=w.group_size, F=w.n_sink_chunks,
                  L=w.n_recent_chunks, Kc=w.top_chunks, Kg=w.top_groups,
                  n_hf=w.n_hf_pairs, theta=w.rope_theta, Hq=w.n_q_heads,
                  Hkv=w.n_kv_heads, d=w.head_dim, period=w.rope_period)


def round_to_cache(x: np.ndarray, dtype: str) -> np.ndarray:
    """The value a rotated-key cache of ``dtype`` holds for float64 x: an
    attention that reads a cache of rotated keys sees them in the model's
    dtype (a bf16 model keeps its keys, rotated, in bf16).  bf16: x rounded
    to 8 significant bits, ties to even; f32: numpy's round-to-nearest;
    f64: x itself."""
    x = np.asarray(x, np.float64)
    if dtype == "f64":
        return x
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    m, e = np.frexp(x)                 # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0) / 256.0, e)  # np.round: half to even


# --------------------------------------------------------------------------
# RoPE (RoFormer, cited by the pages; xllm-io page section 3, Mixed-RoPE)
# --------------------------------------------------------------------------

def rope_inv_freq(d: int, theta: float) -> np.ndarray:
    """theta_i = theta^(-2i/d) for pair i < d/2 (RoFormer frequencies)."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / d)


def high_freq_pair_count(d: int, theta: float, C: int) -> int:
    """Pairs whose wavelength 2*pi/theta_i is below the chunk size C.

    The pages name fast- and slow-rotating pairs without a numeric split;
    reading: a pair is high frequency when it completes a turn inside one
    chunk (strict "<").  Frequencies fall with i, so these are pairs 0..n-1.
    """
    wavelength = 2.0 * np.pi / rope_inv_freq(d, theta)
    return int(np.count_nonzero(wavelength < C))


def rope_position(pos, period: int = 0) -> np.ndarray:
    """The position index RoPE is given for position ``pos``.

    xllm-io page, Sec. 5.5 (interaction with long-context positional
    encoding): the variant that wraps the RoPE position index, p <- p mod
    65536.  ``period`` = 0 keeps absolute positions.  The wrap is applied to
    the value itself, also to a block's fractional middle position; callers
    keep every block inside one period (period % C == 0), so the middle of a
    block is the middle of its wrapped positions.
    """
    pos = np.asarray(pos, dtype=np.float64)
    return np.mod(pos, float(period)) if period else pos


def rope(x: np.ndarray, pos, theta: float, period: int = 0) -> np.ndarray:
    """Rotate x[..., n, d] by R_p at positions pos[n] (may be fractional).

    Pair i is (x[i], x[i + d/2]) (half-split layout, reading of the pages'
    unprinted RoPE); R_p turns it counter-clockwise by p * theta_i, with p
    the position index of ``rope_position`` (wrapped when period > 0).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    ang = np.multiply.outer(rope_position(pos, period), rope_inv_freq(d, theta))
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


# --------------------------------------------------------------------------
# Mixed-RoPE summaries (xllm-io page section 3, summary equation; framework
# paragraph: closed chunks carry one chunk summary and C/g_s group summaries)
# --------------------------------------------------------------------------

def block_summaries(k_raw: np.ndarray, size: int, n_hf: int, theta: float,
                    period: int = 0) -> np.ndarray:
    """Summaries of consecutive complete blocks of ``size`` tokens.

    k_raw [..., n, d] holds raw (pre-RoPE) keys at positions 0..n-1.  For a
    block G with first token f (so |G| = size, middle position
    p_mid = f + (|G|-1)/2, the mean position):
      pairs i <  n_hf: (1/|G|) sum_{j in G} R_j k_j      (rotate, then mean)
      pairs i >= n_hf: R_{p_mid}((1/|G|) sum_{j in G} k_j) (mean, then rotate)
    Only complete blocks are summarised (the pages route over closed chunks).
    Every R_p takes its position through ``rope_position`` (``period``).
    """
    k_raw = np.asarray(k_raw, dtype=np.float64)
    n, d = k_raw.shape[-2], k_raw.shape[-1]
    h = d // 2
    nb = n // size
    k = k_raw[..., : nb * size, :]
    rot_mean = rope(k, np.arange(nb * size), theta, period)
    rot_mean = rot_mean.reshape(*k.shape[:-2], nb, size, d).mean(axis=-2)
    raw_mean = k.reshape(*k.shape[:-2], nb, size, d).mean(axis=-2)
    p_mid = np.arange(nb) * size + (size - 1) / 2.0
    low = rope(raw_mean, p_mid, theta, period)
    out = low.copy()
    hf = np.r_[np.arange(n_hf), h + np.arange(n_hf)].astype(np.int64)
    out[..., hf] = rot_mean[..., hf]
    return out


def summaries(k_raw: np.ndarray, n_tokens: int, p: Params):
    """Chunk and group summaries of the first ``n_tokens`` keys."""
    k = np.asarray(k_raw, dtype=np.float64)[..., :n_tokens, :]
    return (block_summaries(k, p.C, p.n_hf, p.theta, p.period),
            block_summaries(k, p.gs, p.n_hf, p.theta, p.period))


# --------------------------------------------------------------------------
# Routing policy (xllm-io page section 3, routing policy)
# --------------------------------------------------------------------------

def fixed_chunks(t: int, F: int, L: int) -> list:
    """Closed chunks always visible from query chunk t: the first F chunks,
    the last L closed chunks and the immediately previous chunk (forced in
    when it is not already in the recent window).  Set union, sorted."""
    vis = set(range(min(F, t)))
    vis |= set(range(max(0, t - L), t))
    if t >= 1:
        vis.add(t - 1)
    return sorted(vis)


def middle_chunks(t: int, F: int, L: int) -> list:
    """Closed chunks outside the fixed windows: they compete for routing."""
    fixed = set(fixed_chunks(t, F, L))
    return [m for m in range(t) if m not in fixed]


def select_top(ids, scores, k: int):
    """First min(k, len) ids ordered by (score descending, id ascending).

    Returns (selected ids ascending, margin, kth score).  The margin is
    s_(k) - s_(k+1) when more than k candidates compete, else +inf.
    Lowest id wins exact ties.
    """
    ids = np.asarray(ids, dtype=np.int64)
    scores = np.asarray(scores, dtype=np.float64)
    if k <= 0 or ids.size == 0:
        return [], math.inf, math.nan
    order = np.lexsort((ids, -scores))
    kk = min(k, ids.size)
    sel = sorted(int(x) for x in ids[order[:kk]])
    s_k = float(scores[order[kk - 1]])
    margin = float(scores[order[kk - 1]] - scores[order[kk]]) if ids.size > k else math.inf
    return sel, margin, s_k


def unit_queries(t: int, q_pos0: int, n_q: int, C: int) -> np.ndarray:
    """Positions of the queries that fall in query chunk t."""
    lo = max(t * C, q_pos0)
    hi = min((t + 1) * C, q_pos0 + n_q)
    return np.arange(lo, hi)


def query_chunks(q_pos0: int, n_q: int, C: int) -> range:
    return range(q_pos0 // C, (q_pos0 + n_q - 1) // C + 1)


def unit_rows(q_b: np.ndarray, kvh: int, qpos: np.ndarray, q_pos0: int, p: Params) -> np.ndarray:
    """RoPE-rotated query rows (query, head) of one unit, from the raw
    queries q_b [Hq][n_q][d] of one sequence: heads h with h // G == kvh
    (standard GQA).  Returns [G * len(qpos), d]."""
    G = p.Hq // p.Hkv
    raw = np.asarray(q_b[kvh * G:(kvh + 1) * G][:, qpos - q_pos0, :], dtype=np.float64)
    return rope(raw, qpos, p.theta, p.period).reshape(-1, p.d)


def route_unit(rows: np.ndarray, t: int, csum: np.ndarray, gsum: np.ndarray, p: Params) -> dict:
    """Two-level routing for one (sequence, KV head, query chunk t).

    Chunk score s[m] = q^T c_m, aggregated by the max over the unit's query
    rows (query chunk x GQA group; the pages score with one q but route per
    processing block).  M_sel = topK_c over the middle chunks.  With K_g > 0,
    the groups of the chunks in M_sel are scored the same way against the
    group summaries and G_sel = topK_g of them (global group id m*C/g_s + g).
    """
    mids = middle_chunks(t, p.F, p.L)
    out = dict(mid=mids, sel_chunks=[], sel_groups=[], margin_c=math.inf,
               margin_g=math.inf, s_kc=math.nan, s_kg=math.nan,
               chunk_scores=None, group_scores=None, group_cands=[])
    if not mids or p.Kc <= 0 or rows.shape[0] == 0:
        return out
    sc = (rows @ csum[mids].T).max(axis=0)
    selc, mc, skc = select_top(mids, sc, p.Kc)
    out.update(sel_chunks=selc, margin_c=mc, s_kc=skc, chunk_scores=sc)
    if p.Kg > 0 and selc:
        r = p.groups_per_chunk
        cands = [m * r + g for m in selc for g in range(r)]
        sg = (rows @ gsum[cands].T).max(axis=0)
        selg, mg, skg = select_top(cands, sg, p.Kg)
        out.update(sel_groups=selg, margin_g=mg, s_kg=skg, group_scores=sg,
                   group_cands=cands)
    return out


def visible_granules(t: int, q_last: int, sel_chunks, sel_groups, p: Params) -> list:
    """Granules whose exact tokens the unit attends to (sorted, unique):
    the fixed chunks, the routed groups (or the routed chunks whole when
    K_g = 0), and the current chunk's granules up to the last query (the
    causal mask inside it is applied by the attention)."""
    r = p.groups_per_chunk
    gran = set()
    for m in fixed_chunks(t, p.F, p.L):
        gran.update(range(m * r, (m + 1) * r))
    if p.Kg > 0:
        gran.update(sel_groups)
    else:
        for m in sel_chunks:
            gran.update(range(m * r, (m + 1) * r))
    for g in range(t * r, (t + 1) * r):
        if g * p.gs <= q_last:
            gran.add(g)
    return sorted(gran)


def max_granules(p: Params) -> int:
    r = p.groups_per_chunk
    routed = p.Kg if p.Kg > 0 else p.Kc * r
    return r * (1 + p.F + max(p.L, 1)) + routed


def route(q_raw, q_pos0: int, n_q: int, csum, gsum, p: Params, units=None) -> dict:
    """Route every (b, kvh, t) unit (or only ``units``).

    Returns dict with arrays chunk_idx [B,Hkv,NQC,Kc], group_idx
    [B,Hkv,NQC,max(Kg,1)], granules [B,Hkv,NQC,G_max], count [B,Hkv,NQC]
    (index lists ascending, -1 padded) and ``info[(b,kvh,t)]`` with the
    per-unit route_unit() result.  Units not routed hold -1 / 0.
    """
    B = q_raw.shape[0]
    tq = list(query_chunks(q_pos0, n_q, p.C))
    t0 = tq[0]
    nqc = len(tq)
    gmax = max_granules(p)
    ci = np.full((B, p.Hkv, nqc, max(p.Kc, 1)), -1, np.int64)
    gi = np.full((B, p.Hkv, nqc, max(p.Kg, 1)), -1, np.int64)
    gr = np.full((B, p.Hkv, nqc, gmax), -1, np.int64)
    cnt = np.zeros((B, p.Hkv, nqc), np.int64)
    info = {}
    if units is None:
        units = [(b, h, t) for b in range(B) for h in range(p.Hkv) for t in tq]
    for (b, kvh, t) in units:
        qpos = unit_queries(t, q_pos0, n_q, p.C)
        rows = unit_rows(q_raw[b], kvh, qpos, q_pos0, p)
        res = route_unit(rows, t, np.asarray(csum[b, kvh], np.float64),
                         np.asarray(gsum[b, kvh], np.float64) if gsum is not None else None, p)
        gl = visible_granules(t, int(qpos[-1]), res["sel_chunks"], res["sel_groups"], p)
        res["granules"] = gl
        info[(b, kvh, t)] = res
        u = t - t0
        ci[b, kvh, u, :len(res["sel_chunks"])] = res["sel_chunks"]
        gi[b, kvh, u, :len(res["sel_groups"])] = res["sel_groups"]
        gr[b, kvh, u, :len(gl)] = gl
        cnt[b, kvh, u] = len(gl)
    return dict(chunk_idx=ci, group_idx=gi, granules=gr, count=cnt, info=info, t0=t0)


# --------------------------------------------------------------------------
# Exact-token attention (xllm-io page section 3: exact-token output; Eq. 1)
# --------------------------------------------------------------------------

def _softmax_attend(rows, keys, vals, mask, scale):
    """softmax over the True entries of mask[R, nk], max-subtracted, fp64."""
    logits = (rows @ keys.T) * scale
    logits = np.where(mask, logits, -np.inf)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    e = np.where(mask, e, 0.0)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ vals) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def attend_given(q_raw, q_pos0: int, n_q: int, k_raw, v, granules, count, p: Params,
                 t0: int = None, units=None):
    """Softmax attention of every query row over the exact tokens of its
    unit's granule list, with keys j <= i inside the current chunk.

    granules [B,Hkv,NQC,*] / count [B,Hkv,NQC] index units by t - t0.
    Returns out [B,Hq,n_q,d], lse [B,Hq,n_q]; rows of units not listed in
    ``units`` are NaN.
    """
    B = q_raw.shape[0]
    G = p.Hq // p.Hkv
    tq = list(query_chunks(q_pos0, n_q, p.C))
    if t0 is None:
        t0 = tq[0]
    out = np.full(q_raw.shape, np.nan)
    lse = np.full(q_raw.shape[:3], np.nan)
    if units is None:
        units = [(b, h, t) for b in range(B) for h in range(p.Hkv) for t in tq]
    for (b, kvh, t) in units:
        gl = np.asarray(granules[b, kvh, t - t0, : int(count[b, kvh, t - t0])], np.int64)
        tok = (gl[:, None] * p.gs + np.arange(p.gs)[None, :]).reshape(-1)
        kk = round_to_cache(rope(np.asarray(k_raw[b, kvh][tok], np.float64), tok, p.theta, p.period),
                            p.key_cache)
        vv = np.asarray(v[b, kvh][tok], np.float64)
        qpos = unit_queries(t, q_pos0, n_q, p.C)
        mask = (tok[None, :] < t * p.C) | (tok[None, :] <= qpos[:, None])
        for hl in range(G):
            h = kvh * G + hl
            rows = rope(np.asarray(q_raw[b, h, qpos - q_pos0, :], np.float64), qpos, p.theta, p.period)
            o, ls = _softmax_attend(rows, kk, vv, mask, p.softmax_scale)
            out[b, h, qpos - q_pos0] = o
            lse[b, h, qpos - q_pos0] = ls
    return out, lse


def unrope(x: np.ndarray, pos, theta: float, period: int = 0) -> np.ndarray:
    """R_p^T x: the transpose (inverse) rotation, i.e. a turn by -p * theta_i
    with p the (wrapped) position index."""
    return rope(x, -rope_position(pos, period), theta)


def attend_backward(q_raw, q_pos0: int, n_q: int, k_raw, v, granules, count, d_out, p: Params,
                    t0: int = None, units=None):
    """Gradients of exact-token attention over fixed granule lists.

    The routes are a discrete choice and stay fixed (no gradient flows
    through summaries or selection); the gradient is that of the exact-token
    softmax attention of each query row over its visible tokens (xllm-io
    page, section 3, exact-token output; Eq. (1) restricted to the visible
    set), with RoPE applied to the raw q and k.  For one row i with visible
    set V_i, scale s, rotated q~_i, k~_j:
      P_ij = softmax_j(s q~_i . k~_j),  O_i = sum_j P_ij v_j,
      dv_j += P_ij dO_i,  dP_ij = dO_i . v_j,  D_i = dO_i . O_i,
      dS_ij = P_ij (dP_ij - D_i),
      dq~_i = s sum_j dS_ij k~_j,  dk~_j += s dS_ij q~_i,
    and the raw gradients are the transposed rotations dq_i = R_i^T dq~_i,
    dk_j = R_j^T dk~_j.  A KV head's K/V gradients sum over the G query heads
    that read it.  Returns dq [B,Hq,n_q,d], dk, dv [B,Hkv,kv_cap,d] (float64;
    rows of units not listed stay 0).
    """
    q = np.asarray(q_raw, np.float64)
    do = np.asarray(d_out, np.float64)
    B = q.shape[0]
    G = p.Hq // p.Hkv
    tq = list(query_chunks(q_pos0, n_q, p.C))
    if t0 is None:
        t0 = tq[0]
    dq = np.zeros(q.shape)
    dk = np.zeros(np.asarray(k_raw).shape)
    dv = np.zeros(np.asarray(v).shape)
    if units is None:
        units = [(b, h, t) for b in range(B) for h in range(p.Hkv) for t in tq]
    sc = p.softmax_scale
    for (b, kvh, t) in units:
        gl = np.asarray(granules[b, kvh, t - t0, : int(count[b, kvh, t - t0])], np.int64)
        tok = (gl[:, None] * p.gs + np.arange(p.gs)[None, :]).reshape(-1)
        kk = round_to_cache(rope(np.asarray(k_raw[b, kvh][tok], np.float64), tok, p.theta, p.period),
                            p.key_cache)
        vv = np.asarray(v[b, kvh][tok], np.float64)
        qpos = unit_queries(t, q_pos0, n_q, p.C)
        mask = (tok[None, :] < t * p.C) | (tok[None, :] <= qpos[:, None])
        dkk = np.zeros(kk.shape)
        for hl in range(G):
            h = kvh * G + hl
            rows = rope(q[b, h, qpos - q_pos0, :], qpos, p.theta, p.period)
            logits = np.where(mask, (rows @ kk.T) * sc, -np.inf)
            e = np.exp(logits - logits.max(axis=1, keepdims=True))
            P = e / e.sum(axis=1, keepdims=True)
            o = P @ vv
            g = do[b, h, qpos - q_pos0, :]
            dv[b, kvh][tok] += P.T @ g
            dP = g @ vv.T
            D = (g * o).sum(axis=1, keepdims=True)
            dS = P * (dP - D)
            dq[b, h, qpos - q_pos0, :] = unrope(sc * (dS @ kk), qpos, p.theta, p.period)
            dkk += sc * (dS.T @ rows)
        dk[b, kvh][tok] += unrope(dkk, tok, p.theta, p.period)
    return dq, dk, dv


def dense_causal(q_raw, q_pos0: int, n_q: int, k_raw, v, p: Params, heads=None, q_index=None):
    """Eq. (1): each query i attends to every key j <= i (RoPE on q and k).

    ``heads``/``q_index`` restrict the rows computed (others NaN)."""
    q = np.asarray(q_raw, dtype=np.float64)
    B = q.shape[0]
    G = p.Hq // p.Hkv
    out = np.full(q.shape, np.nan)
    lse = np.full(q.shape[:3], np.nan)
    qi = np.arange(n_q) if q_index is None else np.asarray(q_index)
    nk = q_pos0 + int(qi.max()) + 1
    for b in range(B):
        qrot = rope(q[b][:, qi, :], q_pos0 + qi, p.theta, p.period)
        for kvh in range(p.Hkv):
            kk = round_to_cache(rope(np.asarray(k_raw[b, kvh][:nk], np.float64), np.arange(nk), p.theta,
                                     p.period), p.key_cache)
            vv = np.asarray(v[b, kvh][:nk], np.float64)
            mask = np.arange(nk)[None, :] <= (q_pos0 + qi)[:, None]
            for hl in range(G):
                h = kvh * G + hl
                if heads is not None and h not in heads:
                    continue
                o, ls = _softmax_attend(qrot[h], kk, vv, mask, p.softmax_scale)
                out[b, h, qi] = o
                lse[b, h, qi] = ls
    return out, lse


# --------------------------------------------------------------------------
# Eq. (2): token-attention cost
# --------------------------------------------------------------------------

def visible_token_count(granule_lists: dict, q_pos0: int, n_q: int, p: Params) -> int:
    """Sum over query tokens i of |V_i| for one (sequence, KV head), from the
    per-chunk granule lists {t: [granules]} (keys j <= i inside chunk t)."""
    total = 0
    for t, gl in granule_lists.items():
        tok = (np.asarray(gl, np.int64)[:, None] * p.gs + np.arange(p.gs)).reshape(-1)
        for i in unit_queries(t, q_pos0, n_q, p.C):
            total += int(np.count_nonzero((tok < t * p.C) | (tok <= i)))
    return total


def visible_token_count_closed_form(q_pos0: int, n_q: int, p: Params) -> int:
    """Sum_t [rows_t * (|Fixed(t)| C + routed_t) + sum_i (i - tC + 1)], with
    routed_t = g_s * min(K_g, (C/g_s) min(K_c, |Mid(t)|)) when K_g > 0, else
    C * min(K_c, |Mid(t)|)."""
    total = 0
    r = p.groups_per_chunk
    for t in query_chunks(q_pos0, n_q, p.C):
        qpos = unit_queries(t, q_pos0, n_q, p.C)
        nmid = len(middle_chunks(t, p.F, p.L))
        nsel = min(p.Kc, nmid) if p.Kc > 0 else 0
        routed = p.gs * min(p.Kg, r * nsel) if p.Kg > 0 else p.C * nsel
        fixed = len(fixed_chunks(t, p.F, p.L)) * p.C
        total += len(qpos) * (fixed + routed) + int(np.sum(qpos - t * p.C + 1))
    return total


def eq2_bound(n: int, p: Params) -> int:
    """n * (C + (F + L) C + B_route) with B_route = K_g g_s or K_c C."""
    b_route = p.Kg * p.gs if p.Kg > 0 else p.Kc * p.C
    return n * (p.C + (p.F + p.L) * p.C + b_route)
