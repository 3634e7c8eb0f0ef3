"""Seeded random shapes for parity sweeps: chunk and group sizes, sink and
recent windows, chunk and group budgets, GQA ratio, head size, dtype,
ragged query starts and RoPE wraps drawn inside the documented limits
(g_s | C <= 64, C * G <= 512 query rows per unit, d in {64, 128}), at sizes
the oracle handles in seconds.  Shared by the CPU check that every drawn
shape is accepted by the library's sizing calls and by the GPU parity sweep.
"""
from __future__ import annotations

import numpy as np

import workloads as W

N_CONFIGS = 40


def random_workload(i: int) -> W.Workload:
    rng = np.random.default_rng(7100 + i)
    d = int(rng.choice([64, 128]))
    C = int(rng.choice([16, 32, 64]))
    gs = int(rng.choice([g for g in (2, 4, 8, 16, 32) if g <= C]))
    G = int(rng.choice([g for g in (1, 2, 4, 8) if C * g <= 512]))
    hkv = int(rng.choice([1, 2]))
    r = C // gs
    kc = int(rng.integers(0, 7))
    # K_g: whole chunks (0), fewer groups than the chosen chunks hold, or more
    kg = int(rng.choice([0, max(1, kc * r // 2), kc * r + 3])) if kc > 0 else 0
    n_ctx = int(rng.integers(150, 1200))
    extra = int(rng.choice([0, C]))
    kv_cap = (n_ctx + C - 1) // C * C + extra
    q_pos0 = int(rng.choice([0, int(rng.integers(1, n_ctx - 1))]))
    period = int(rng.choice([0, C * int(rng.integers(2, 9))]))
    return W.Workload(
        name=f"random_{i}", batch=int(rng.integers(1, 3)), n_q_heads=hkv * G, n_kv_heads=hkv,
        head_dim=d, n_ctx=n_ctx, kv_cap=kv_cap, q_pos0=q_pos0, n_q=n_ctx - q_pos0,
        dtype=str(rng.choice(["bf16", "bf16", "f32"])), rope_theta=float(rng.choice([1e4, 1e6])),
        chunk_size=C, group_size=gs, n_sink_chunks=int(rng.integers(0, 4)),
        n_recent_chunks=int(rng.integers(0, 4)), top_chunks=kc, top_groups=kg,
        n_hf_pairs=int(rng.integers(0, d // 2 + 1)), planted=0, seed_offset=40 + i,
        rope_period=period)


N_DECODE = 12


def random_decode_workload(i: int) -> W.Workload:
    """One query per sequence at the end of a long context (up to a few
    hundred middle chunks, so that some draws take the segmented scoring and
    all of them the split-key decode attention)."""
    rng = np.random.default_rng(9300 + i)
    d = int(rng.choice([64, 128]))
    C = int(rng.choice([16, 32, 64]))
    gs = int(rng.choice([g for g in (2, 4, 8, 16, 32) if g <= C]))
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 4]))
    r = C // gs
    kc = int(rng.integers(1, 9))
    kg = min(256, int(rng.choice([0, max(1, kc * r // 2), kc * r + 2])))  # routing selects <= 256
    n_ctx = int(rng.integers(100, 420)) * C + int(rng.integers(1, C + 1))
    kv_cap = (n_ctx + C - 1) // C * C + int(rng.choice([0, C]))
    period = int(rng.choice([0, C * int(rng.integers(8, 64))]))
    return W.Workload(
        name=f"random_decode_{i}", batch=int(rng.integers(1, 5)), n_q_heads=hkv * G,
        n_kv_heads=hkv, head_dim=d, n_ctx=n_ctx, kv_cap=kv_cap, q_pos0=n_ctx - 1, n_q=1,
        dtype="bf16", rope_theta=float(rng.choice([1e4, 1e7])), chunk_size=C, group_size=gs,
        n_sink_chunks=int(rng.integers(0, 4)), n_recent_chunks=int(rng.integers(0, 9)),
        top_chunks=kc, top_groups=kg, n_hf_pairs=int(rng.integers(0, d // 2 + 1)), planted=0,
        seed_offset=90 + i, rope_period=period)


N_STREAM = 8


def random_stream_workload(i: int):
    """(workload, cache_slots) of a streaming decode session: one query per
    step for n_q steps after a prefix of q_pos0 tokens (bf16, at most 16
    rows per unit); the cache is the smallest allowed or a roomy one."""
    import hierarchical_kv_routing_amd as H
    rng = np.random.default_rng(11500 + i)
    d = int(rng.choice([64, 128]))
    C = int(rng.choice([16, 32, 64]))
    gs = int(rng.choice([g for g in (2, 4, 8, 16, 32) if g <= C]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    hkv = int(rng.choice([1, 2]))
    r = C // gs
    kc = int(rng.integers(1, 7))
    kg = min(256, int(rng.choice([0, max(1, kc * r // 2), kc * r + 2])))  # routing selects <= 256
    prefix = int(rng.integers(20, 120)) * C  # sessions start at a chunk boundary
    steps = int(rng.integers(C // 2, 2 * C + 8))
    kv_cap = (prefix + steps + C - 1) // C * C + int(rng.choice([0, C]))
    period = int(rng.choice([0, C * int(rng.integers(4, 32))]))
    w = W.Workload(
        name=f"random_stream_{i}", batch=int(rng.integers(1, 3)), n_q_heads=hkv * G,
        n_kv_heads=hkv, head_dim=d, n_ctx=prefix + steps, kv_cap=kv_cap, q_pos0=prefix, n_q=steps,
        dtype="bf16", rope_theta=float(rng.choice([1e4, 1e7])), chunk_size=C, group_size=gs,
        n_sink_chunks=int(rng.integers(0, 3)), n_recent_chunks=int(rng.integers(0, 4)),
        top_chunks=kc, top_groups=kg, n_hf_pairs=int(rng.integers(0, d // 2 + 1)), planted=0,
        seed_offset=130 + i, rope_period=period)
    need = w.batch * w.n_kv_heads * H.max_granules(H.Config.from_workload(w))
    cache = need if rng.integers(0, 2) == 0 else 3 * need
    return w, cache
