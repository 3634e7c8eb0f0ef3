"""Seeded synthetic workloads for routed exact-token attention (HGA).

This module is shared by the CPU oracle and the HIP path as the single source
of inputs.  It holds sizes, budgets and random numbers only: no RoPE, no
summaries, no scores, no routing and no attention arithmetic.

Input recipe (one independent PCG64 stream per (tensor, batch, head) slab, so
that a test can regenerate one slab without drawing the others):

* Q, K, V are standard normals drawn in float32, laid out [B][H][n][d].
* ``key_rank > 0`` gives each KV head a low-rank key structure:
  K = sqrt(1/2) * Z @ W + sqrt(1/2) * E with Z ~ N(0,1)^(n x r),
  W ~ N(0, 1/r)^(r x d) (one W per KV head) and E iid N(0,1).
* Planted long-range matches: a unit vector u, supported on the two lowest
  RoPE frequency pairs (dims d/2-2, d/2-1, d-2, d-1), is added with amplitude
  a (a^2 = 8 sqrt(d), i.e. +8 sigma of an N(0,1) dot product of length d) to a
  raw query row i and a raw key row j whose chunk lies past the sink chunks
  and before the recent window of i's chunk.  On those pairs a RoPE rotation
  by the distance turns u by at most ~0.7 rad for the listed workloads, so the
  planted dot product stays large after rotation.
* bf16 workloads round the float32 draws to bfloat16 with round-to-nearest-
  even; both sides then see exactly the same values.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

BASE_SEED = 260630709

KIND_Q, KIND_K, KIND_V, KIND_Z, KIND_W, KIND_E, KIND_PLANT = range(7)


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_ctx: int            # tokens whose K/V exist (positions 0 .. n_ctx-1)
    kv_cap: int           # allocated K/V slots per (batch, kv head)
    q_pos0: int           # position of the first query
    n_q: int              # number of query tokens
    dtype: str            # "f32" or "bf16"
    rope_theta: float
    chunk_size: int       # C
    group_size: int       # g_s
    n_sink_chunks: int    # F
    n_recent_chunks: int  # L
    top_chunks: int       # K_c
    top_groups: int       # K_g (0 = whole routed chunks are opened)
    n_hf_pairs: int       # RoPE pairs [0, n_hf) are the high-frequency ones
    planted: int          # planted matches per (batch, kv head)
    planted_per_q_head: int = 0   # decode: planted matches per (batch, query head)
    key_rank: int = 0
    seed_offset: int = 0
    rope_period: int = 0  # RoPE positions wrap modulo this (0 = absolute)

    @property
    def group_ratio(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads.  n_hf_pairs follows the rule "wavelength 2*pi/theta_i
# below C": 9 pairs for d=64, theta=1e4 and 10 pairs for d=128, theta=1e7.
TINY_F32 = Workload(
    name="tiny_f32_n1024", batch=1, n_q_heads=1, n_kv_heads=1, head_dim=64,
    n_ctx=1024, kv_cap=1024, q_pos0=0, n_q=1024, dtype="f32", rope_theta=1e4,
    chunk_size=64, group_size=16, n_sink_chunks=2, n_recent_chunks=2,
    top_chunks=4, top_groups=4, n_hf_pairs=9, planted=4, seed_offset=1)

SMALLLM_PREFILL = Workload(
    name="smalllm_prefill_b4_h8_n4096", batch=4, n_q_heads=8, n_kv_heads=8,
    head_dim=64, n_ctx=4096, kv_cap=4096, q_pos0=0, n_q=4096, dtype="bf16",
    rope_theta=1e4, chunk_size=64, group_size=16, n_sink_chunks=2,
    n_recent_chunks=8, top_chunks=8, top_groups=16, n_hf_pairs=9, planted=32,
    seed_offset=2)

QWEN3_PREFILL = Workload(
    name="qwen3_prefill_h32kv4_n32768", batch=1, n_q_heads=32, n_kv_heads=4,
    head_dim=128, n_ctx=32768, kv_cap=32768, q_pos0=0, n_q=32768,
    dtype="bf16", rope_theta=1e7, chunk_size=64, group_size=16,
    n_sink_chunks=2, n_recent_chunks=8, top_chunks=16, top_groups=32,
    n_hf_pairs=10, planted=64, key_rank=8, seed_offset=3)

DECODE_64K = Workload(
    name="decode_b16_h32kv4_ctx65536", batch=16, n_q_heads=32, n_kv_heads=4,
    head_dim=128, n_ctx=65537, kv_cap=65536 + 64, q_pos0=65536, n_q=1,
    dtype="bf16", rope_theta=1e7, chunk_size=64, group_size=16,
    n_sink_chunks=2, n_recent_chunks=8, top_chunks=8, top_groups=16,
    n_hf_pairs=10, planted=0, planted_per_q_head=1, seed_offset=4)

HOST_TIERED_CHUNK = Workload(
    name="host_tiered_chunk_only_n131072", batch=1, n_q_heads=32,
    n_kv_heads=4, head_dim=128, n_ctx=131072, kv_cap=131072, q_pos0=0,
    n_q=131072, dtype="bf16", rope_theta=1e7, chunk_size=64, group_size=16,
    n_sink_chunks=2, n_recent_chunks=8, top_chunks=24, top_groups=0,
    n_hf_pairs=10, planted=64, key_rank=8, seed_offset=5)

HOST_TIERED_GROUP = HOST_TIERED_CHUNK.scaled(
    name="host_tiered_chunk_group_n131072", top_chunks=16, top_groups=32)

ALL = (TINY_F32, SMALLLM_PREFILL, QWEN3_PREFILL, DECODE_64K,
       HOST_TIERED_CHUNK, HOST_TIERED_GROUP)


def _rng(w: Workload, seed: int, kind: int, b: int, h: int) -> np.random.Generator:
    ss = np.random.SeedSequence([BASE_SEED + w.seed_offset, seed, kind, b, h])
    return np.random.Generator(np.random.PCG64(ss))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> float32 holding the nearest bfloat16 (ties to even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) & np.uint32(0xFFFF0000)).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 values that are exact bfloat16 -> their uint16 bit patterns."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _finish(w: Workload, x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32, copy=False)
    return round_to_bf16(x) if w.dtype == "bf16" else x


def _plant_vector(w: Workload, rng: np.random.Generator) -> np.ndarray:
    d = w.head_dim
    h = d // 2
    dims = np.array([h - 2, h - 1, d - 2, d - 1])
    u = np.zeros(d)
    g = rng.standard_normal(4)
    u[dims] = g / np.linalg.norm(g)
    return u


def plants(w: Workload, seed: int, b: int, kvh: int):
    """Planted matches touching KV head ``kvh`` of sequence ``b``.

    Returns a list of (query_head, query_pos, key_pos, vector) with the
    vector already scaled by the amplitude a, a^2 = 8 sqrt(d).
    """
    rng = _rng(w, seed, KIND_PLANT, b, kvh)
    C, F, L = w.chunk_size, w.n_sink_chunks, max(w.n_recent_chunks, 1)
    amp = np.sqrt(8.0 * np.sqrt(w.head_dim))
    q_lo, q_hi = w.q_pos0, w.q_pos0 + w.n_q
    out = []
    heads = []
    if w.planted_per_q_head:
        for hl in range(w.group_ratio):
            heads += [kvh * w.group_ratio + hl] * w.planted_per_q_head
    else:
        heads = [kvh * w.group_ratio + int(rng.integers(w.group_ratio))
                 for _ in range(w.planted)]
    # queries must sit in a chunk that has keys beyond the sinks and before
    # the recent window: chunk index >= F + L + 1
    first_ok = max(q_lo, (F + L + 1) * C)
    if first_ok >= q_hi:
        return []
    for hq in heads:
        i = int(rng.integers(first_ok, q_hi))
        ti = i // C
        j_lo, j_hi = F * C, (ti - L) * C
        j = int(rng.integers(j_lo, j_hi))
        out.append((hq, i, j, amp * _plant_vector(w, rng)))
    return out


def k_slab(w: Workload, seed: int, b: int, kvh: int, with_plants: bool = True) -> np.ndarray:
    """Raw (pre-RoPE) keys of one (batch, kv head): float32 [kv_cap, d]."""
    n, d = w.n_ctx, w.head_dim
    if w.key_rank:
        r = w.key_rank
        z = _rng(w, seed, KIND_Z, b, kvh).standard_normal((n, r), dtype=np.float32)
        wm = _rng(w, seed, KIND_W, 0, kvh).standard_normal((r, d), dtype=np.float32) / np.sqrt(r)
        e = _rng(w, seed, KIND_E, b, kvh).standard_normal((n, d), dtype=np.float32)
        k = np.sqrt(0.5) * (z.astype(np.float64) @ wm.astype(np.float64)) + np.sqrt(0.5) * e
    else:
        k = _rng(w, seed, KIND_K, b, kvh).standard_normal((n, d), dtype=np.float32)
    k = np.asarray(k, dtype=np.float64)
    if with_plants:
        for (_, _, j, vec) in plants(w, seed, b, kvh):
            k[j] += vec
    out = np.zeros((w.kv_cap, d), dtype=np.float32)
    out[:n] = _finish(w, k)
    return out


def v_slab(w: Workload, seed: int, b: int, kvh: int) -> np.ndarray:
    n, d = w.n_ctx, w.head_dim
    out = np.zeros((w.kv_cap, d), dtype=np.float32)
    out[:n] = _finish(w, _rng(w, seed, KIND_V, b, kvh).standard_normal((n, d), dtype=np.float32))
    return out


def q_slab(w: Workload, seed: int, b: int, hq: int) -> np.ndarray:
    """Raw (pre-RoPE) queries of one (batch, query head): float32 [n_q, d]."""
    q = _rng(w, seed, KIND_Q, b, hq).standard_normal((w.n_q, w.head_dim), dtype=np.float32)
    q = q.astype(np.float64)
    kvh = hq // w.group_ratio
    for (h, i, _, vec) in plants(w, seed, b, kvh):
        if h == hq:
            q[i - w.q_pos0] += vec
    return _finish(w, q)


def make_inputs(w: Workload, seed: int = 0, threads: int = 1):
    """Whole tensors: q [B,Hq,n_q,d], k [B,Hkv,kv_cap,d], v [B,Hkv,kv_cap,d]
    (float32; bf16 workloads hold exact bfloat16 values).  Slabs are
    independent streams, so ``threads`` > 1 gives the same values."""
    from concurrent.futures import ThreadPoolExecutor
    B, Hq, Hkv, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    q = np.empty((B, Hq, w.n_q, d), dtype=np.float32)
    k = np.empty((B, Hkv, w.kv_cap, d), dtype=np.float32)
    v = np.empty((B, Hkv, w.kv_cap, d), dtype=np.float32)
    jobs = []
    for b in range(B):
        for h in range(Hq):
            jobs.append((q, b, h, q_slab))
        for h in range(Hkv):
            jobs.append((k, b, h, k_slab))
            jobs.append((v, b, h, v_slab))

    def run(job):
        arr, b, h, fn = job
        arr[b, h] = fn(w, seed, b, h)

    if threads <= 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(run, jobs))
    return q, k, v


def plant_list(w: Workload, seed: int = 0):
    """All planted matches as (b, query_head, query_pos, key_pos)."""
    out = []
    for b in range(w.batch):
        for kvh in range(w.n_kv_heads):
            for (hq, i, j, _) in plants(w, seed, b, kvh):
                out.append((b, hq, i, j))
    return out
