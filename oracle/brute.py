"""Pure-Python brute force of HGA for tiny inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Written with plain
loops over tokens, pairs and keys and ``math`` scalars, independently of the
vectorised ``hga_ref``, so that an indexing or broadcasting mistake in one of
them shows up as a disagreement.  Visibility is materialised as an explicit
per-query set of key positions (the n x n mask), routing uses a full
``sorted`` of (-score, id), and attention a per-row two-pass softmax.

Inputs are nested lists or NumPy arrays of floats; outputs are Python lists.
Rules followed: xllm-io paper-review page, section 3 (framework paragraph,
Mixed-RoPE summary equation, routing policy, selection equation, exact-token
output, Eq. 1).
"""
from __future__ import annotations

import math


def _freq(i, d, theta):
    return float(theta) ** (-2.0 * i / d)


def wrap(pos, period):
    """RoPE position index: pos itself, or pos taken modulo ``period`` for the
    wrapped-position variant (xllm-io page, Sec. 5.5)."""
    if not period:
        return pos
    return pos - period * math.floor(pos / period)


def rotate(vec, pos, theta, period=0):
    """R_pos on a d-vector: pair (vec[i], vec[i + d/2]) turned by p*theta_i,
    p = wrap(pos, period)."""
    pos = wrap(pos, period)
    d = len(vec)
    h = d // 2
    out = [0.0] * d
    for i in range(h):
        a = pos * _freq(i, d, theta)
        c, s = math.cos(a), math.sin(a)
        x, y = float(vec[i]), float(vec[i + h])
        out[i] = x * c - y * s
        out[i + h] = x * s + y * c
    return out


def block_summary(keys, first, n_hf, theta, period=0):
    """Summary of the block of raw keys ``keys`` whose first position is first.

    With wrapped positions the block's middle is the middle of its wrapped
    positions (a block never straddles a multiple of the period)."""
    size = len(keys)
    d = len(keys[0])
    h = d // 2
    rot_sum = [0.0] * d
    raw_sum = [0.0] * d
    for j in range(size):
        r = rotate(keys[j], first + j, theta, period)
        for e in range(d):
            rot_sum[e] += r[e]
            raw_sum[e] += float(keys[j][e])
    p_mid = wrap(first, period) + (size - 1) / 2.0
    low = rotate([x / size for x in raw_sum], p_mid, theta)
    out = list(low)
    for i in range(n_hf):
        out[i] = rot_sum[i] / size
        out[i + h] = rot_sum[i + h] / size
    return out


def all_summaries(keys, n_tokens, size, n_hf, theta, period=0):
    return [block_summary([keys[j] for j in range(b * size, (b + 1) * size)], b * size, n_hf, theta,
                          period)
            for b in range(n_tokens // size)]


def visible_chunks_fixed(t, F, L):
    out = []
    for m in range(t):
        sink = m < F
        recent = t - L <= m
        prev = m == t - 1
        if sink or recent or prev:
            out.append(m)
    return out


def dot(a, b):
    s = 0.0
    for x, y in zip(a, b):
        s += float(x) * float(y)
    return s


def topk(cands, score_of, k):
    ranked = sorted(cands, key=lambda c: (-score_of[c], c))
    return sorted(ranked[:k])


def route_one(rows, t, chunk_sums, group_sums, C, gs, F, L, Kc, Kg):
    """rows: rotated query rows of the unit.  Returns (chunks, groups)."""
    fixed = visible_chunks_fixed(t, F, L)
    mids = [m for m in range(t) if m not in fixed]
    if not mids or Kc <= 0 or not rows:
        return [], []
    cs = {m: max(dot(r, chunk_sums[m]) for r in rows) for m in mids}
    selc = topk(mids, cs, Kc)
    if Kg <= 0:
        return selc, []
    per = C // gs
    cands = [m * per + g for m in selc for g in range(per)]
    gsc = {c: max(dot(r, group_sums[c]) for r in rows) for c in cands}
    return selc, topk(cands, gsc, Kg)


def visible_keys(i, t, selc, selg, C, gs, F, L, Kg):
    """Key positions visible to the query at position i in chunk t."""
    keys = set()
    for m in visible_chunks_fixed(t, F, L):
        keys.update(range(m * C, (m + 1) * C))
    if Kg > 0:
        for g in selg:
            keys.update(range(g * gs, (g + 1) * gs))
    else:
        for m in selc:
            keys.update(range(m * C, (m + 1) * C))
    keys.update(range(t * C, i + 1))
    return sorted(keys)


def attend_row(qrot, keys_rot, vals, visible, scale):
    logits = [dot(qrot, keys_rot[j]) * scale for j in visible]
    m = max(logits)
    w = [math.exp(x - m) for x in logits]
    z = sum(w)
    d = len(vals[0])
    out = [0.0] * d
    for wt, j in zip(w, visible):
        for e in range(d):
            out[e] += wt * float(vals[j][e])
    return [x / z for x in out], m + math.log(z)


def routed_attention(q, k, v, q_pos0, C, gs, F, L, Kc, Kg, n_hf, theta, Hq, Hkv, scale=None,
                     period=0):
    """Whole pipeline for one sequence: q [Hq][n_q][d], k, v [Hkv][n][d].

    Summaries are taken over the closed chunks before each query chunk.
    Returns (out [Hq][n_q][d], routes {(kvh, t): (chunks, groups)}).
    """
    d = len(q[0][0])
    n_q = len(q[0])
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    n_tok = q_pos0 + n_q
    routes = {}
    out = [[None] * n_q for _ in range(Hq)]
    for kvh in range(Hkv):
        keys_rot = [rotate(k[kvh][j], j, theta, period) for j in range(n_tok)]
        csum = all_summaries(k[kvh], n_tok, C, n_hf, theta, period)
        gsum = all_summaries(k[kvh], n_tok, gs, n_hf, theta, period)
        for t in range(q_pos0 // C, (n_tok - 1) // C + 1):
            qs = [i for i in range(max(t * C, q_pos0), min((t + 1) * C, n_tok))]
            rows = [rotate(q[kvh * G + hl][i - q_pos0], i, theta, period) for hl in range(G) for i in qs]
            selc, selg = route_one(rows, t, csum, gsum, C, gs, F, L, Kc, Kg)
            routes[(kvh, t)] = (selc, selg)
            for hl in range(G):
                h = kvh * G + hl
                for i in qs:
                    vis = visible_keys(i, t, selc, selg, C, gs, F, L, Kg)
                    o, _ = attend_row(rotate(q[h][i - q_pos0], i, theta, period), keys_rot, v[kvh], vis,
                                      scale)
                    out[h][i - q_pos0] = o
    return out, routes


def dense_attention(q, k, v, q_pos0, theta, Hq, Hkv, scale=None, period=0):
    d = len(q[0][0])
    n_q = len(q[0])
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = [[None] * n_q for _ in range(Hq)]
    for h in range(Hq):
        kvh = h // G
        keys_rot = [rotate(k[kvh][j], j, theta, period) for j in range(q_pos0 + n_q)]
        for qi in range(n_q):
            i = q_pos0 + qi
            o, _ = attend_row(rotate(q[h][qi], i, theta, period), keys_rot, v[kvh], list(range(i + 1)),
                              scale)
            out[h][qi] = o
    return out
