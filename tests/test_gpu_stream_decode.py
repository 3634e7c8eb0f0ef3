"""Streaming decode from the host tier (DecodeSession) against the
device-resident path: every step's output and LSE bit for bit, the session's
summaries and host store after the appends, with a roomy cache and with the
smallest allowed one (evictions on every step); and the routes and outputs
of sampled steps against the oracle (the pages' "cache vs no cache" and
"decode vs recompute" checks, xllm-io page, Tab. 7)."""
import numpy as np
import pytest

import hierarchical_kv_routing_amd as H
import workloads as W
from tests import parity as P
from tests.random_configs import N_STREAM, random_stream_workload

pytestmark = pytest.mark.gpu

PREFIX = 4096
STEPS = 140   # crosses a chunk boundary; the closed chunk is routed later (L = 1)
CAP = PREFIX + 192


def _workload(**kw):
    base = dict(batch=2, n_ctx=PREFIX + STEPS, kv_cap=CAP, q_pos0=PREFIX, n_q=STEPS,
                n_recent_chunks=1, planted=0, planted_per_q_head=1)
    base.update(kw)
    return W.DECODE_64K.scaled(**base)


def _reference(run, w, dev):
    """Device-resident route + attend of every step's query (and its routes)."""
    import torch
    cfg = run.cfg
    outs, lses, routes = [], [], []
    for s in range(w.n_q):
        pos = w.q_pos0 + s
        q = run.q[:, :, s:s + 1].contiguous()
        ro = H.route_outputs(cfg, w.batch, pos, 1, dev)
        H.route(cfg, q, pos, run.csum, run.gsum, w.kv_cap, ro["chunk_idx"], ro["group_idx"],
                ro["granules"], ro["granule_count"], ro["workspace"])
        aw = H.attend_workspace_bytes(cfg, w.batch, pos, 1)
        ws = torch.empty(max(aw, 16), dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        H.attend(cfg, q, pos, run.k_rot, run.v, ro["granules"], ro["granule_count"], out, lse, ws)
        outs.append(out)
        lses.append(lse)
        routes.append(ro)
    torch.cuda.synchronize()
    return outs, lses, routes


class _StepRun:
    """The arrays parity.compare_routes / check_attention read, for one
    decode step (one query per sequence at position pos)."""

    def __init__(self, w, pos, ro, out, lse):
        self.w = w.scaled(q_pos0=pos, n_q=1, n_ctx=pos + 1)
        self.arrays = {n: ro[n].cpu().numpy() for n in ("chunk_idx", "group_idx", "granules",
                                                        "granule_count")}
        self.arrays["out"] = out.float().cpu().numpy()
        self.arrays["lse"] = lse.float().cpu().numpy()

    def np(self, name):
        return self.arrays[name]


def _oracle_steps(w, q, k, v, routes, outs, lses, steps):
    """The session's routes and outputs at the given steps against the
    oracle (own summaries of the tokens up to each step's position, routes
    of that one query, attention on the step's granule lists)."""
    for s in steps:
        pos = w.q_pos0 + s
        run = _StepRun(w, pos, routes[s], outs[s], lses[s])
        qs = np.ascontiguousarray(q[:, :, s:s + 1])
        units = P.all_units(run.w)
        orc = P.oracle_route(run, qs, k, units)
        exact, near = P.compare_routes(run, orc, units, name=f"stream:{w.name}:step{s}")
        assert exact + near == len(units)
        P.check_attention(run, qs, k, v, units, name=f"stream:{w.name}:step{s}")


def _session_run(run, w, cache_slots, dev, poison=False, with_stats=True):
    import torch
    cfg = run.cfg
    # store and summary tables hold only the prefix; the session appends the rest
    prefix = w.q_pos0
    k_rot = run.k_rot.clone()
    v = run.v.clone()
    k_rot[:, :, prefix:] = 0
    v[:, :, prefix:] = 0
    store = H.host_store(cfg, k_rot, v)
    csum = run.csum.clone()
    gsum = run.gsum.clone()
    csum[:, :, prefix // cfg.chunk_size:] = 0
    gsum[:, :, prefix // cfg.group_size:] = 0
    sess = H.DecodeSession(cfg, w.batch, w.kv_cap, prefix, cache_slots, store, device=dev)
    if poison:
        # the session may not rely on its device buffer's contents: all bits
        # set reads as NaN in every float format
        sess.dev.fill_(255)
    outs, lses, stats = [], [], []
    for s in range(w.n_q):
        pos = w.q_pos0 + s
        sess.append(run.k[:, :, pos:pos + 1].contiguous(), run.v[:, :, pos:pos + 1].contiguous(),
                    pos, csum, gsum)
        q = run.q[:, :, s:s + 1].contiguous()
        out = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
        stats.append(sess.step(q, pos, csum, gsum, out, lse, stats=with_stats))
        outs.append(out)
        lses.append(lse)
    torch.cuda.synchronize()
    sess.close()
    return outs, lses, stats, csum, gsum, store


def _check_session(w, cache_slots, poison=False, seed=0, with_stats=True):
    """Session outputs vs the device path at every step, then its summaries
    and host store vs a prefill build; returns the per-step stats."""
    import torch
    dev = torch.device("cuda:0")
    q, k, v = P.make_inputs_parallel(w, seed)
    run = P.DeviceRun(w, q, k, v, route=False, attend=False)
    ref_out, ref_lse, ref_routes = _reference(run, w, dev)
    outs, lses, stats, csum, gsum, store = _session_run(run, w, cache_slots, dev, poison=poison,
                                                        with_stats=with_stats)
    bad = [s for s in range(w.n_q)
           if not (torch.equal(outs[s], ref_out[s]) and torch.equal(lses[s], ref_lse[s]))]
    detail = []
    for s in bad[:3]:
        do = (outs[s].float() - ref_out[s].float()).abs()
        dl = (lses[s] - ref_lse[s]).abs()
        rows = torch.nonzero(do.amax(dim=-1) > 0).tolist()
        detail.append(f"step {s}: max|dO| {do.max().item():.3g} max|dlse| {dl.max().item():.3g} "
                      f"nan {int(torch.isnan(outs[s]).sum())} rows {rows[:8]} "
                      + (f"copied {stats[s]['granules_copied']} hits {stats[s]['granules_hit']}"
                         if stats[s] is not None else ""))
    assert not bad, f"steps differing from the device path: {bad[:10]}; " + "; ".join(detail)
    end = w.q_pos0 + w.n_q
    n_closed = end // run.cfg.chunk_size
    assert torch.equal(csum[:, :, :n_closed], run.csum[:, :, :n_closed])
    ng_closed = end // run.cfg.group_size
    assert torch.equal(gsum[:, :, :ng_closed], run.gsum[:, :, :ng_closed])
    ref_store = H.host_store(run.cfg, run.k_rot, run.v)
    ng = (end + run.cfg.group_size - 1) // run.cfg.group_size
    got = store[:, :, :ng].reshape(w.batch, w.n_kv_heads, -1, w.head_dim)
    want = ref_store[:, :, :ng].reshape(w.batch, w.n_kv_heads, -1, w.head_dim)
    # token rows [0, end) of both halves (K, V)
    g = run.cfg.group_size
    sel = np.arange(ng * 2 * g).reshape(ng, 2, g)
    tok = (np.arange(ng)[:, None, None] * g + np.arange(g)[None, None, :]).repeat(2, axis=1)
    rows = sel[tok < end]
    assert torch.equal(got[:, :, rows], want[:, :, rows])
    # the session's steps (bitwise the device path's) against the oracle:
    # the first step, the step that closes the first chunk and the one after
    # it, a middle one and the last
    C = run.cfg.chunk_size
    close = (C - 1 - w.q_pos0 % C) % C
    steps = sorted({0, min(close, w.n_q - 1), min(close + 1, w.n_q - 1), w.n_q // 2, w.n_q - 1})
    _oracle_steps(w, q, k, v, ref_routes, outs, lses, steps)
    return stats


@pytest.mark.parametrize("cache", ["roomy", "smallest", "smallest_poisoned"])
def test_stream_decode_equals_device_path(cache):
    w = _workload()
    print(f"[gpu] stream decode ({cache}): {w}", flush=True)
    need = w.batch * w.n_kv_heads * H.max_granules(H.Config.from_workload(w))
    slots = 4 * need if cache == "roomy" else need
    stats = _check_session(w, slots, poison=cache.endswith("poisoned"))
    copied = [st["granules_copied"] for st in stats]
    hits = [st["granules_hit"] for st in stats]
    print(f"[gpu] stream decode ({cache}): copied first {copied[0]} then mean "
          f"{np.mean(copied[1:]):.1f}, hits mean {np.mean(hits[1:]):.1f}", flush=True)
    assert copied[0] > 0 and hits[0] == 0
    if cache == "roomy":
        # later steps find the fixed windows (and any repeated routes) in the
        # cache: only the granule being filled and new routes are copied
        # (the synthetic queries are independent, so routes change a lot)
        assert np.mean(copied[1:]) < 0.5 * copied[0]
        assert min(hits[1:]) > 0


@pytest.mark.parametrize("cache", ["roomy", "smallest"])
def test_stream_decode_unsynchronised(cache):
    """Steps enqueued back to back with no host wait between them (no stats
    asked): the cache lookup, the gathers and the attention stay ordered on
    the stream, and every step equals the device path bit for bit."""
    w = _workload()
    print(f"[gpu] stream decode unsynchronised ({cache}): {w}", flush=True)
    need = w.batch * w.n_kv_heads * H.max_granules(H.Config.from_workload(w))
    stats = _check_session(w, 4 * need if cache == "roomy" else need, with_stats=False)
    assert all(st is None for st in stats)


@pytest.mark.parametrize("i", range(N_STREAM))
def test_stream_decode_random_shapes(i):
    """Random streaming shapes (chunk / group sizes, windows, budgets, GQA
    ratio, d, prefix length, steps crossing chunk boundaries, RoPE wrap,
    the smallest or a roomy cache): every step bit for bit equal to the
    device path."""
    w, cache = random_stream_workload(i)
    print(f"[gpu] stream decode random {i}: {w} cache {cache}", flush=True)
    _check_session(w, cache, seed=i)
