"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test names the passage it follows (xllm-io paper-review page of
arXiv:2606.30709, section 3, unless stated otherwise).  None of them
compares the oracle with itself: the checks are closed forms, values printed
on the pages or derived by hand from their rules (tests/golden/), a library
routine (torch SDPA), textbook identities, or the independent brute force.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import brute
from oracle import hga_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- RoPE ----

def test_rope_matches_complex_rotation():
    """R_p on pair i equals multiplying x_i + i x_{i+d/2} by exp(i p theta_i)
    with theta_i = theta^(-2i/d) (RoFormer, cited by the pages)."""
    d, theta = 16, 1e4
    x = _rand((5, d), 1)
    pos = np.array([0.0, 1.0, 7.5, 1000.0, 65536.0])
    z = x[:, : d // 2] + 1j * x[:, d // 2:]
    freqs = np.array([theta ** (-2.0 * i / d) for i in range(d // 2)])
    zr = z * np.exp(1j * pos[:, None] * freqs[None, :])
    want = np.concatenate([zr.real, zr.imag], axis=1)
    np.testing.assert_allclose(R.rope(x, pos, theta), want, rtol=0, atol=1e-12)


def test_rope_relative_position_and_norm():
    """<R_i q, R_j k> depends on j - i only; rotations keep the norm."""
    d, theta = 32, 1e7
    q, k = _rand((1, d), 2), _rand((1, d), 3)
    a = float((R.rope(q, [100.0], theta) @ R.rope(k, [37.0], theta).T)[0, 0])
    b = float((R.rope(q, [163.0], theta) @ R.rope(k, [100.0], theta).T)[0, 0])
    assert abs(a - b) < 1e-10
    y = R.rope(_rand((4, d), 4), [1.0, 2.0, 3.0, 4.0], theta)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(_rand((4, d), 4), axis=1), rtol=1e-13)


def test_rope_brute_agrees():
    d, theta = 12, 1e4
    x = _rand((3, d), 5)
    pos = [3.0, 17.5, 900.0]
    want = np.array([brute.rotate(x[i], pos[i], theta) for i in range(3)])
    np.testing.assert_allclose(R.rope(x, pos, theta), want, atol=1e-12)


def test_high_frequency_split_closed_form():
    """Wavelength 2 pi theta^(2i/d) below C = 64, from log10 by hand:
    d=64, theta=1e4: theta^(2*8/64) = 10^1 -> 62.83 < 64, theta^(18/64) =
    10^1.125 -> 83.8 > 64, so 9 pairs.  d=128, theta=1e7: 10^(7*18/128) =
    9.65 -> 60.6 < 64, 10^(7*20/128) = 12.4 -> 78.0 > 64, so 10 pairs."""
    assert 2 * math.pi * 10 ** 1.0 < 64 < 2 * math.pi * 10 ** 1.125
    assert 2 * math.pi * 10 ** (7 * 18 / 128) < 64 < 2 * math.pi * 10 ** (7 * 20 / 128)
    assert R.high_freq_pair_count(64, 1e4, 64) == 9
    assert R.high_freq_pair_count(128, 1e7, 64) == 10
    for w in W.ALL:
        assert w.n_hf_pairs == R.high_freq_pair_count(w.head_dim, w.rope_theta, w.chunk_size)


# ----------------------------------------------------------- summaries ----

@pytest.mark.parametrize("n_hf", [0, 3, 8])
def test_summary_single_token_is_rotated_key(n_hf):
    """With C = g_s = 1 every summary is the RoPE-rotated key (both branches
    of the Mixed-RoPE equation reduce to R_j k_j)."""
    d, theta, n = 16, 1e4, 40
    k = _rand((2, 3, n, d), 6)
    s = R.block_summaries(k, 1, n_hf, theta)
    want = np.stack([brute.rotate(k[0, 0, j], j, theta) for j in range(n)])
    np.testing.assert_allclose(s[0, 0], want, atol=1e-12)


def test_summary_all_high_and_all_low():
    """n_hf = d/2: mean of rotated keys; n_hf = 0: R_{p_mid}(mean raw key)."""
    d, theta, size = 8, 1e4, 4
    k = _rand((12, d), 7)
    s_hi = R.block_summaries(k, size, d // 2, theta)
    s_lo = R.block_summaries(k, size, 0, theta)
    for b in range(3):
        rot = np.mean([brute.rotate(k[b * size + j], b * size + j, theta) for j in range(size)], axis=0)
        np.testing.assert_allclose(s_hi[b], rot, atol=1e-12)
        mid = b * size + (size - 1) / 2
        np.testing.assert_allclose(s_lo[b], brute.rotate(k[b * size: (b + 1) * size].mean(0), mid, theta), atol=1e-12)


def test_summary_constant_key_dirichlet_closed_form():
    """A constant raw key k over a block of s tokens starting at f:
    high-frequency pair i -> D_s(theta_i) R_{p_mid} k with
    D_s(a) = sin(s a / 2) / (s sin(a / 2)) (geometric sum of e^{i j a});
    low-frequency pair -> R_{p_mid} k exactly."""
    d, theta, size, n_hf = 16, 1e4, 16, 5
    kvec = _rand((d,), 8)
    k = np.tile(kvec, (3 * size, 1))
    s = R.block_summaries(k, size, n_hf, theta)
    h = d // 2
    for b in range(3):
        mid = b * size + (size - 1) / 2
        base = brute.rotate(kvec, mid, theta)
        for i in range(h):
            a = theta ** (-2.0 * i / d)
            f = math.sin(size * a / 2) / (size * math.sin(a / 2)) if i < n_hf else 1.0
            assert abs(s[b, i] - f * base[i]) < 1e-12
            assert abs(s[b, i + h] - f * base[i + h]) < 1e-12


def test_summary_brute_agrees_and_is_linear():
    d, theta, n = 8, 1e4, 48
    k1, k2 = _rand((n, d), 9), _rand((n, d), 10)
    for size, n_hf in ((16, 2), (4, 3), (8, 0)):
        s = R.block_summaries(k1, size, n_hf, theta)
        want = np.array(brute.all_summaries(k1, n, size, n_hf, theta))
        np.testing.assert_allclose(s, want, atol=1e-12)
        lin = R.block_summaries(2.0 * k1 - 3.0 * k2, size, n_hf, theta)
        np.testing.assert_allclose(lin, 2.0 * s - 3.0 * R.block_summaries(k2, size, n_hf, theta), atol=1e-11)


def test_summary_only_closed_blocks():
    k = _rand((70, 8), 11)
    c, g = R.summaries(k, 70, R.Params(C=32, gs=8, F=0, L=0, Kc=0, Kg=0, n_hf=1, theta=1e4, Hq=1, Hkv=1, d=8))
    assert c.shape == (2, 8) and g.shape == (8, 8)


# ------------------------------------------------------------- routing ----

def test_visibility_rules_golden():
    fx = _load("visibility_rules.json")
    for case in fx["cases"]:
        assert R.fixed_chunks(case["t"], case["F"], case["L"]) == case["fixed"], case
        assert R.middle_chunks(case["t"], case["F"], case["L"]) == case["middle"], case
        assert brute.visible_chunks_fixed(case["t"], case["F"], case["L"]) == case["fixed"], case


def test_route_handmade_golden():
    fx = _load("route_handmade.json")
    pr, ex = fx["params"], fx["expected"]
    p = R.Params(C=pr["C"], gs=pr["gs"], F=pr["F"], L=pr["L"], Kc=pr["Kc"], Kg=pr["Kg"],
                 n_hf=0, theta=1e4, Hq=1, Hkv=1, d=pr["d"])
    rows = np.array(fx["rows"], float)
    cs, gsum = np.array(fx["chunk_sums"], float), np.array(fx["group_sums"], float)
    res = R.route_unit(rows, pr["t"], cs, gsum, p)
    assert res["mid"] == ex["middle"]
    np.testing.assert_array_equal(res["chunk_scores"], ex["chunk_scores"])
    assert res["sel_chunks"] == ex["sel_chunks"]
    assert res["margin_c"] == ex["margin_c"]
    assert res["sel_groups"] == ex["sel_groups"]
    assert res["margin_g"] == ex["margin_g"]
    assert R.visible_granules(pr["t"], pr["q_last"], res["sel_chunks"], res["sel_groups"], p) == ex["granules"]
    assert R.visible_granules(pr["t"], 24, res["sel_chunks"], res["sel_groups"], p) == ex["granules_q_last_24"]
    p0 = R.Params(**{**p.__dict__, "Kg": 0})
    res0 = R.route_unit(rows, pr["t"], cs, gsum, p0)
    assert R.visible_granules(pr["t"], pr["q_last"], res0["sel_chunks"], [], p0) == ex["granules_chunk_only"]
    bc, bg = brute.route_one([list(r) for r in rows], pr["t"], cs.tolist(), gsum.tolist(),
                             pr["C"], pr["gs"], pr["F"], pr["L"], pr["Kc"], pr["Kg"])
    assert bc == ex["sel_chunks"] and bg == ex["sel_groups"]


def test_route_fewer_candidates_than_budget_and_zero_budget():
    p = R.Params(C=4, gs=2, F=1, L=1, Kc=10, Kg=3, n_hf=0, theta=1e4, Hq=1, Hkv=1, d=4)
    rows = _rand((3, 4), 12)
    cs, gsum = _rand((8, 4), 13), _rand((16, 4), 14)
    res = R.route_unit(rows, 6, cs, gsum, p)
    assert res["sel_chunks"] == [1, 2, 3, 4] and res["margin_c"] == math.inf
    assert len(res["sel_groups"]) == 3
    p0 = R.Params(**{**p.__dict__, "Kc": 0})
    res0 = R.route_unit(rows, 6, cs, gsum, p0)
    assert res0["sel_chunks"] == [] and res0["sel_groups"] == []


def _tiny_workload(**kw):
    base = dict(name="tiny", batch=2, n_q_heads=4, n_kv_heads=2, head_dim=8,
                n_ctx=96, kv_cap=96, q_pos0=0, n_q=96, dtype="f32", rope_theta=1e4,
                chunk_size=8, group_size=4, n_sink_chunks=1, n_recent_chunks=2,
                top_chunks=2, top_groups=3, n_hf_pairs=2, planted=2, seed_offset=77)
    base.update(kw)
    return W.Workload(**base)


def _brute_pipeline(w, q, k, v, b):
    return brute.routed_attention(
        q[b].tolist(), k[b].tolist(), v[b].tolist(), w.q_pos0, w.chunk_size, w.group_size,
        w.n_sink_chunks, w.n_recent_chunks, w.top_chunks, w.top_groups, w.n_hf_pairs,
        w.rope_theta, w.n_q_heads, w.n_kv_heads)


def _oracle_pipeline(w, q, k, v):
    # exact keys: the brute force it is checked against rotates in float64
    p = dataclasses.replace(R.params_from_workload(w), key_cache="f64")
    cs, gsum = R.summaries(k, w.q_pos0 + w.n_q, p)
    rt = R.route(q, w.q_pos0, w.n_q, cs, gsum, p)
    out, lse = R.attend_given(q, w.q_pos0, w.n_q, k, v, rt["granules"], rt["count"], p, t0=rt["t0"])
    return p, rt, out, lse


@pytest.mark.parametrize("kw", [
    {},
    dict(top_groups=0),
    dict(n_recent_chunks=0, n_sink_chunks=0),
    dict(q_pos0=37, n_q=59, n_ctx=96),
    dict(chunk_size=4, group_size=4, top_groups=1),
])
def test_pipeline_matches_brute_force(kw):
    w = _tiny_workload(**kw)
    q, k, v = W.make_inputs(w, seed=3)
    p, rt, out, _ = _oracle_pipeline(w, q, k, v)
    for b in range(w.batch):
        bout, routes = _brute_pipeline(w, q, k, v, b)
        for (kvh, t), (selc, selg) in routes.items():
            info = rt["info"][(b, kvh, t)]
            assert info["sel_chunks"] == selc and info["sel_groups"] == selg
        np.testing.assert_allclose(out[b], np.array(bout), atol=1e-12)


def test_route_invariant_to_query_scale():
    w = _tiny_workload(n_ctx=160, kv_cap=160, n_q=160)
    q, k, _ = W.make_inputs(w, seed=4)
    p = R.params_from_workload(w)
    cs, gsum = R.summaries(k, 160, p)
    a = R.route(q, 0, 160, cs, gsum, p)
    b = R.route(3.7 * q.astype(np.float64), 0, 160, cs, gsum, p)
    np.testing.assert_array_equal(a["granules"], b["granules"])


def test_route_exact_tie_lowest_index_wins():
    p = R.Params(C=4, gs=2, F=0, L=1, Kc=2, Kg=1, n_hf=0, theta=1e4, Hq=1, Hkv=1, d=4)
    rows = np.array([[1.0, 0, 0, 0]])
    cs = np.tile([[2.0, 0, 0, 0]], (10, 1))
    gsum = np.tile([[1.0, 0, 0, 0]], (20, 1))
    res = R.route_unit(rows, 9, cs, gsum, p)
    assert res["sel_chunks"] == [0, 1] and res["sel_groups"] == [0]
    assert res["margin_c"] == 0.0


def test_planted_dominant_key_is_routed():
    """A single key made dominant (large dot product with one query of the
    chunk) puts its chunk into M_sel and its group into G_sel."""
    w = _tiny_workload(batch=1, n_q_heads=1, n_kv_heads=1, head_dim=16, n_ctx=256, kv_cap=256,
                       n_q=256, chunk_size=16, group_size=4, n_sink_chunks=1, n_recent_chunks=1,
                       top_chunks=1, top_groups=1, n_hf_pairs=3, planted=0)
    q, k, v = W.make_inputs(w, seed=5)
    q = q.astype(np.float64)
    k = k.astype(np.float64)
    i, j = 250, 70                # query chunk 15, key chunk 4 (middle), group 17
    u = np.zeros(16)
    u[[7, 15]] = 1 / math.sqrt(2)  # lowest-frequency pair: barely turns over 180 tokens
    q[0, 0, i] += 12 * u
    k[0, 0, j] += 12 * u
    p = R.params_from_workload(w)
    cs, gsum = R.summaries(k, 256, p)
    rt = R.route(q, 0, 256, cs, gsum, p)
    info = rt["info"][(0, 0, 15)]
    assert info["sel_chunks"] == [4] and info["sel_groups"] == [17]


# ----------------------------------------------------------- attention ----

def _sdpa_causal(q, k, v, p):
    torch = pytest.importorskip("torch")
    G = p.Hq // p.Hkv
    n = q.shape[2]
    qr = torch.from_numpy(R.rope(q.astype(np.float64), np.arange(n), p.theta))
    kr = torch.from_numpy(R.rope(k[:, :, :n].astype(np.float64), np.arange(n), p.theta))
    vv = torch.from_numpy(v[:, :, :n].astype(np.float64))
    kr = kr.repeat_interleave(G, dim=1)
    vv = vv.repeat_interleave(G, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(qr, kr, vv, is_causal=True).numpy()


@pytest.mark.parametrize("kw", [dict(top_groups=0), dict(top_groups=64)])
def test_full_coverage_equals_dense_causal_and_sdpa(kw):
    """With budgets covering every middle chunk, routed exact-token attention
    equals dense causal attention, Eq. (1) (the pages' repository check
    'router, full coverage vs causal SDPA', Table 7).  Dense is in turn
    pinned to torch's fp64 SDPA with is_causal."""
    w = _tiny_workload(n_ctx=128, kv_cap=128, n_q=128, top_chunks=16, **kw)
    q, k, v = W.make_inputs(w, seed=6)
    p, rt, out, lse = _oracle_pipeline(w, q, k, v)
    dense, dlse = R.dense_causal(q, 0, 128, k, v, p)
    np.testing.assert_allclose(out, dense, atol=1e-12)
    np.testing.assert_allclose(lse, dlse, atol=1e-12)
    np.testing.assert_allclose(dense, _sdpa_causal(q, k, v, p), atol=1e-12)
    bd = brute.dense_attention(q[0].tolist(), k[0].tolist(), v[0].tolist(), 0, w.rope_theta, w.n_q_heads, w.n_kv_heads)
    np.testing.assert_allclose(dense[0], np.array(bd), atol=1e-12)


def test_value_shift_and_band_pattern():
    """V + c shifts every output by c; K_c = 0 leaves the sink/local pattern,
    checked against an explicitly built mask."""
    w = _tiny_workload(top_chunks=0, top_groups=0, n_ctx=96, n_q=96)
    q, k, v = W.make_inputs(w, seed=7)
    p, rt, out, _ = _oracle_pipeline(w, q, k, v)
    _, _, out2, _ = _oracle_pipeline(w, q, k, v.astype(np.float64) + 0.75)
    np.testing.assert_allclose(out2, out + 0.75, atol=1e-12)
    C, F, L = w.chunk_size, w.n_sink_chunks, w.n_recent_chunks
    n = 96
    mask = np.zeros((n, n), bool)
    for i in range(n):
        t = i // C
        for j in range(i + 1):
            m = j // C
            mask[i, j] = m == t or m < F or m >= t - L or m == t - 1
    qr = R.rope(q[0, 0].astype(np.float64), np.arange(n), p.theta)
    kr = R.rope(k[0, 0, :n].astype(np.float64), np.arange(n), p.theta)
    lg = np.where(mask, qr @ kr.T / math.sqrt(p.d), -np.inf)
    e = np.exp(lg - lg.max(1, keepdims=True))
    want = (e / e.sum(1, keepdims=True)) @ v[0, 0, :n]
    np.testing.assert_allclose(out[0, 0], want, atol=1e-12)


# ------------------------------------- wrapped RoPE positions (Sec. 5.5) ----
# xllm-io page, Sec. 5.5: a variant feeds RoPE the position index modulo
# 65536.  Every position that enters a rotation (queries, keys, and the
# blocks' middle positions of the Mixed-RoPE summaries) is wrapped; causality
# and routing keep absolute positions.


def _prerotate(x, pos, period, theta):
    """Turn pair i of x[..., n, d] by -period * floor(pos / period) * theta_i,
    done as a complex product (independent of the oracle's rope)."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    h = d // 2
    freq = float(theta) ** (-2.0 * np.arange(h) / d)
    shift = -period * np.floor(np.asarray(pos, np.float64) / period)
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * np.multiply.outer(shift, freq))
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("kw", [
    dict(rope_period=32),
    dict(rope_period=16, top_groups=0),
    dict(rope_period=24, q_pos0=37, n_q=59, n_ctx=96),
])
def test_wrapped_pipeline_matches_brute_force(kw):
    """Summaries, routes and outputs with wrapped positions: the vectorised
    oracle (np.mod of every position, fractional middles included) against
    the brute force (floor-based wrap; a block's middle taken from its
    wrapped first position)."""
    w = _tiny_workload(**kw)
    q, k, v = W.make_inputs(w, seed=11)
    p, rt, out, _ = _oracle_pipeline(w, q, k, v)
    for b in range(w.batch):
        bout, routes = brute.routed_attention(
            q[b].tolist(), k[b].tolist(), v[b].tolist(), w.q_pos0, w.chunk_size, w.group_size,
            w.n_sink_chunks, w.n_recent_chunks, w.top_chunks, w.top_groups, w.n_hf_pairs,
            w.rope_theta, w.n_q_heads, w.n_kv_heads, period=w.rope_period)
        for (kvh, t), (selc, selg) in routes.items():
            info = rt["info"][(b, kvh, t)]
            assert info["sel_chunks"] == selc and info["sel_groups"] == selg
        np.testing.assert_allclose(out[b], np.array(bout), atol=1e-12)


@pytest.mark.parametrize("kw", [
    dict(rope_period=32),
    dict(rope_period=64, chunk_size=16, group_size=4, n_ctx=300, kv_cap=304, n_q=300,
         head_dim=16, n_hf_pairs=3, top_chunks=3, top_groups=5),
])
def test_wrap_equals_prerotated_absolute(kw):
    """R_{p mod P} = R_p R_{-P floor(p/P)}: wrapping the positions equals
    absolute positions applied to inputs turned back by whole periods.  A
    block lies inside one period, so its raw mean is turned by the same
    angle as its tokens; summaries, routes, outputs and LSE must agree."""
    w = _tiny_workload(**kw)
    q, k, v = W.make_inputs(w, seed=12)
    P_ = w.rope_period
    qpos = w.q_pos0 + np.arange(w.n_q)
    q2 = _prerotate(q, qpos, P_, w.rope_theta)
    k2 = _prerotate(k, np.arange(w.kv_cap), P_, w.rope_theta)
    p, rt, out, lse = _oracle_pipeline(w, q, k, v)
    w0 = w.scaled(rope_period=0)
    p0, rt0, out0, lse0 = _oracle_pipeline(w0, q2, k2, v)
    cs, gsum = R.summaries(k, w.n_ctx, p)
    cs0, gsum0 = R.summaries(k2, w.n_ctx, p0)
    np.testing.assert_allclose(cs, cs0, atol=1e-12)
    np.testing.assert_allclose(gsum, gsum0, atol=1e-12)
    np.testing.assert_array_equal(rt["granules"], rt0["granules"])
    np.testing.assert_allclose(out, out0, atol=1e-12)
    np.testing.assert_allclose(lse, lse0, atol=1e-12)
    # and the wrap matters: absolute positions on the raw inputs differ
    _, _, out_abs, _ = _oracle_pipeline(w0, q, k, v)
    assert np.abs(out_abs - out).max() > 1e-3


def test_wrap_beyond_context_is_absolute():
    """A period at or beyond every position leaves the path unchanged."""
    w = _tiny_workload(rope_period=96)
    q, k, v = W.make_inputs(w, seed=13)
    _, rt, out, lse = _oracle_pipeline(w, q, k, v)
    _, rt0, out0, lse0 = _oracle_pipeline(w.scaled(rope_period=0), q, k, v)
    np.testing.assert_array_equal(rt["granules"], rt0["granules"])
    assert np.array_equal(out, out0) and np.array_equal(lse, lse0)


def test_wrapped_dense_pattern_by_hand():
    """Dense causal attention with wrapped positions: a query and a key in
    the same period see their true distance; a key one period back is seen
    at the same in-period offset as a key of the query's own period."""
    d, theta, P_ = 8, 1e4, 16
    p = R.Params(C=8, gs=4, F=0, L=0, Kc=0, Kg=0, n_hf=0, theta=theta, Hq=1, Hkv=1, d=d,
                 period=P_)
    rng = np.random.default_rng(14)
    q = rng.standard_normal((1, 1, 40, d))
    k = np.tile(rng.standard_normal(d), (1, 1, 40, 1))  # one key vector at every slot
    v = rng.standard_normal((1, 1, 40, d))
    out, lse = R.dense_causal(q, 0, 40, k, v, p)
    # closed form for row i: logit_j = q_i . R_{(j mod P) - (i mod P)} k / sqrt(d)
    for i in (3, 17, 39):
        z = q[0, 0, i, : d // 2] + 1j * q[0, 0, i, d // 2:]
        kz = k[0, 0, 0, : d // 2] + 1j * k[0, 0, 0, d // 2:]
        freq = theta ** (-2.0 * np.arange(d // 2) / d)
        lg = np.array([np.real(np.sum(np.conj(z) * kz *
                                      np.exp(1j * ((j % P_) - (i % P_)) * freq)))
                       for j in range(i + 1)]) / math.sqrt(d)
        wts = np.exp(lg - lg.max())
        ref = (wts[:, None] * v[0, 0, : i + 1]).sum(0) / wts.sum()
        np.testing.assert_allclose(out[0, 0, i], ref, atol=1e-12)
        np.testing.assert_allclose(lse[0, 0, i], lg.max() + math.log(wts.sum()), atol=1e-12)


# ------------------------------------------------------------ backward ----
# Gradients of exact-token attention with the routes held fixed.


def _loss_and_grads(w, q, k, v, seed):
    p, rt, out, _ = _oracle_pipeline(w, q, k, v)
    do = np.random.default_rng(seed).standard_normal(out.shape)
    dq, dk, dv = R.attend_backward(q, w.q_pos0, w.n_q, k, v, rt["granules"], rt["count"], do, p,
                                   t0=rt["t0"])

    def loss(qq, kk, vv):
        o, _ = R.attend_given(qq, w.q_pos0, w.n_q, kk, vv, rt["granules"], rt["count"], p, t0=rt["t0"])
        return float((o * do).sum())
    return loss, dq, dk, dv


@pytest.mark.parametrize("kw", [{}, dict(top_groups=0, q_pos0=21, n_q=75), dict(rope_period=32)])
def test_backward_matches_finite_differences(kw):
    """dL/dq, dL/dk, dL/dv of L = sum(dO * O) against central differences of
    the oracle's forward (fp64, h = 1e-6), at random coordinates, including
    keys seen through routed groups, sinks and the current chunk."""
    w = _tiny_workload(**kw)
    q, k, v = W.make_inputs(w, seed=21)
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    loss, dq, dk, dv = _loss_and_grads(w, q, k, v, seed=22)
    rng = np.random.default_rng(23)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        n_tok = w.q_pos0 + w.n_q if name != "q" else w.n_q
        for _ in range(8):
            idx = (int(rng.integers(x.shape[0])), int(rng.integers(x.shape[1])),
                   int(rng.integers(n_tok)), int(rng.integers(x.shape[3])))
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, g[idx])


def test_backward_full_coverage_matches_torch_autograd():
    """With budgets covering every middle chunk the routed backward is the
    dense causal backward: torch fp64 autograd through its own RoPE (complex
    rotation) and SDPA with is_causal gives the same raw-input gradients."""
    torch = pytest.importorskip("torch")
    w = _tiny_workload(n_ctx=128, kv_cap=128, n_q=128, top_chunks=16, top_groups=64)
    q, k, v = W.make_inputs(w, seed=24)
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    _, dq, dk, dv = _loss_and_grads(w, q, k, v, seed=25)
    do = np.random.default_rng(25).standard_normal(q.shape)
    G = w.n_q_heads // w.n_kv_heads
    d = w.head_dim
    freq = torch.tensor(w.rope_theta ** (-2.0 * np.arange(d // 2) / d), dtype=torch.float64)
    pos = torch.arange(128, dtype=torch.float64)
    rot = torch.polar(torch.ones(128, d // 2, dtype=torch.float64), pos[:, None] * freq[None, :])

    def rope_t(x):
        z = torch.complex(x[..., : d // 2], x[..., d // 2:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(
        rope_t(qt), rope_t(kt).repeat_interleave(G, dim=1), vt.repeat_interleave(G, dim=1), is_causal=True)
    (o * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-10)


# ---------------------------------------------------------------- Eq. 2 ----

@pytest.mark.parametrize("kw", [{}, dict(top_groups=0), dict(q_pos0=21, n_q=75), dict(n_recent_chunks=0)])
def test_eq2_count_matches_closed_form(kw):
    """The attended-token count of the routed visible sets equals the count
    implied by Eq. (2)'s terms (current chunk causal, F + L fixed chunks,
    routed budget), and stays below n (C + (F+L)C + B_route)."""
    w = _tiny_workload(n_ctx=96, kv_cap=96, **kw)
    q, k, v = W.make_inputs(w, seed=8)
    p, rt, _, _ = _oracle_pipeline(w, q, k, v)
    for b in range(w.batch):
        for kvh in range(w.n_kv_heads):
            gl = {t: info["granules"] for (bb, hh, t), info in rt["info"].items() if bb == b and hh == kvh}
            cnt = R.visible_token_count(gl, w.q_pos0, w.n_q, p)
            assert cnt == R.visible_token_count_closed_form(w.q_pos0, w.n_q, p)
            if w.n_recent_chunks > 0:
                assert cnt <= R.eq2_bound(w.n_q, p)


def test_sparsity_matches_pages():
    fx = _load("sparsity_pages.json")
    for key in ("group", "chunk_only"):
        v = fx[key]
        p = R.Params(C=fx["C"], gs=fx["gs"], F=fx["F"], L=fx["L"], Kc=v["Kc"], Kg=v["Kg"],
                     n_hf=0, theta=1e4, Hq=1, Hkv=1, d=2)
        n = fx["n"]
        t = (n - 1) // p.C
        nsel = min(p.Kc, len(R.middle_chunks(t, p.F, p.L)))
        sel_chunks = R.middle_chunks(t, p.F, p.L)[:nsel]
        r = p.groups_per_chunk
        sel_groups = [m * r + g for m in sel_chunks for g in range(r)][: p.Kg]
        gl = R.visible_granules(t, n - 1, sel_chunks, sel_groups, p)
        vis = R.visible_token_count({t: gl}, n - 1, 1, p)
        assert abs(vis / n - v["printed_fraction"]) <= v["tolerance"], (key, vis)


def test_max_granules_bound():
    for w in W.ALL:
        p = R.params_from_workload(w)
        t = (w.q_pos0 + w.n_q - 1) // w.chunk_size
        nmid = len(R.middle_chunks(t, p.F, p.L))
        r = p.groups_per_chunk
        routed = min(p.Kg, r * min(p.Kc, nmid)) if p.Kg else r * min(p.Kc, nmid)
        assert len(R.fixed_chunks(t, p.F, p.L)) * r + r + routed <= R.max_granules(p)


def test_cache_rounding_is_round_to_nearest_even():
    """round_to_cache("bf16") against torch's float32 -> bfloat16 conversion
    (round to nearest, ties to even) on float32-exact values, including exact
    halfway cases; "f32" against numpy's float64 -> float32 conversion."""
    import torch
    rng = np.random.default_rng(5)
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    bits = x32.view(np.uint32)
    half = ((bits & ~np.uint32(0xFFFF)) | np.uint32(0x8000)).view(np.float32)  # exact ties
    x = np.concatenate([x32, half, -half, np.float32([0.0, 1.0, -2.5, 3.0e38])]).astype(np.float64)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(R.round_to_cache(x, "bf16"), want)
    y = rng.standard_normal(1000) * 1e3
    np.testing.assert_array_equal(R.round_to_cache(y, "f32"), y.astype(np.float32).astype(np.float64))
    np.testing.assert_array_equal(R.round_to_cache(y, "f64"), y)


def _eq2_by_arithmetic(n, C, gs, F, L, Kc, Kg):
    """Eq. (2)'s count for a full prefill of n tokens, from the per-chunk
    min() expressions of tests/golden/eq2_counts.json (no sets, no oracle)."""
    total = 0
    for t in range(n // C):
        fixed = min(t, F + L)
        mid = max(0, t - F - L)
        routed = gs * min(Kg, (C // gs) * min(Kc, mid)) if Kg else C * min(Kc, mid)
        total += C * (C * fixed + routed) + C * (C + 1) // 2
    return total


@pytest.mark.parametrize("case", _load("eq2_counts.json")["cases"], ids=lambda c: c["name"])
def test_eq2_counts_at_the_workloads(case):
    """Eq. (2) at the five benchmark workloads: the hand-derived counts of
    tests/golden/eq2_counts.json equal (a) the per-chunk arithmetic,
    (b) the count over the oracle's own visible sets (fixed windows, a
    full-size routed selection, causal current chunk) at the full length, and
    (c) the oracle's closed form; each stays below n (C + (F+L)C + B_route)."""
    w = {x.name: x for x in W.ALL}[case["name"]]
    p = R.params_from_workload(w)
    assert (p.F, p.L, p.Kc, p.Kg, w.n_q, p.C, p.gs) == (case["F"], case["L"], case["Kc"], case["Kg"],
                                                        case["n"], 64, 16)
    assert _eq2_by_arithmetic(case["n"], 64, 16, case["F"], case["L"], case["Kc"], case["Kg"]) == case["count"]
    r = p.groups_per_chunk
    lists = {}
    for t in range(case["n"] // p.C):
        mids = R.middle_chunks(t, p.F, p.L)
        # any selection of the right size gives the same count: take the
        # highest-index middle chunks and the last groups of the candidates
        sel = mids[len(mids) - min(p.Kc, len(mids)):]
        cands = [m * r + g for m in sel for g in range(r)]
        groups = cands[len(cands) - min(p.Kg, len(cands)):] if p.Kg else []
        lists[t] = R.visible_granules(t, (t + 1) * p.C - 1, sel, groups, p)
    assert R.visible_token_count(lists, 0, case["n"], p) == case["count"]
    assert R.visible_token_count_closed_form(0, case["n"], p) == case["count"]
    assert case["count"] <= R.eq2_bound(case["n"], p) == case["bound"]


def test_eq2_decode_step_count():
    """The decode step (one query at position 65536, the current chunk holding
    only that token) sees 1 + (F+L)C + K_g g_s = 897 tokens (Eq. 2 for one
    query)."""
    fx = _load("eq2_counts.json")["decode"]
    w = W.DECODE_64K
    p = R.params_from_workload(w)
    t = fx["pos"] // p.C
    mids = R.middle_chunks(t, p.F, p.L)
    sel = mids[: p.Kc]
    groups = [m * p.groups_per_chunk + g for m in sel for g in range(p.groups_per_chunk)][: p.Kg]
    gl = R.visible_granules(t, fx["pos"], sel, groups, p)
    assert R.visible_token_count({t: gl}, fx["pos"], 1, p) == fx["count"]
    assert R.visible_token_count_closed_form(fx["pos"], 1, p) == fx["count"]
