"""GPU tests of the pinned-host K/V tier: its outputs equal the device-resident
route + attend path bit for bit (same granules, same order), and match the
oracle on sampled units."""
import numpy as np
import pytest

import hierarchical_kv_routing_amd as H
import workloads as W
from tests import parity as P
from tests.random_configs import N_CONFIGS, random_workload

pytestmark = pytest.mark.gpu


def run_host_tier(run, max_window_chunks, slots, threads=4, copy_stream=True, cache_slots=0):
    import torch
    w, cfg = run.w, run.cfg
    store = H.host_store(cfg, run.k_rot, run.v)
    dt = P.torch_dtype(w)
    dev_b, host_b = H.host_tiered_buffer_bytes(cfg, dt, w.batch, w.q_pos0, w.n_q,
                                               max_window_chunks, slots, cache_slots)
    dev = torch.empty(dev_b, dtype=torch.uint8, device="cuda:0")
    host = torch.empty(host_b, dtype=torch.uint8, pin_memory=True)
    out = torch.full_like(run.out, float("nan"))
    lse = torch.full_like(run.lse, float("nan"))
    xs = torch.cuda.Stream() if copy_stream else None
    stats = H.attend_host_tiered(cfg, run.q, w.q_pos0, store, run.k.shape[2], run.csum, run.gsum,
                                 out, lse, dev, host, max_window_chunks, slots, threads,
                                 copy_stream=xs, cache_slots=cache_slots)
    torch.cuda.synchronize()
    return out, lse, stats


@pytest.mark.parametrize("base", ["chunk_only", "group"])
def test_host_tier_equals_device_path(base):
    import torch
    w0 = W.HOST_TIERED_CHUNK if base == "chunk_only" else W.HOST_TIERED_GROUP
    w = w0.scaled(n_ctx=4096, kv_cap=4096, n_q=4096, planted=16)
    q, k, v = P.make_inputs_parallel(w)
    run = P.DeviceRun(w, q, k, v)
    gmax = H.max_granules(run.cfg)
    slots = w.batch * w.n_kv_heads * gmax + 64    # windows split on slot capacity
    out, lse, stats = run_host_tier(run, max_window_chunks=16, slots=slots)
    print(f"[gpu] host tier {base}: {stats}", flush=True)
    assert stats["windows"] > 64 // 16
    total = int(run.np("granule_count").sum())
    assert 0 < stats["granules_copied"] <= total
    same = (bool(torch.equal(out, run.out)), bool(torch.equal(lse, run.lse)))
    assert all(same), same
    units = P.sample_units(w, 6)
    P.check_attention(run, q, k, v, units, out=out.float().cpu().numpy(), lse=lse.cpu().numpy())


@pytest.mark.parametrize("base", ["chunk_only", "group"])
def test_warm_tier_equals_device_path(base):
    """A warm tier small enough to evict: same outputs bit for bit, fewer
    granules copied than without it, and the reuse counted."""
    import torch
    w0 = W.HOST_TIERED_CHUNK if base == "chunk_only" else W.HOST_TIERED_GROUP
    w = w0.scaled(n_ctx=4096, kv_cap=4096, n_q=4096, planted=16)
    q, k, v = P.make_inputs_parallel(w)
    run = P.DeviceRun(w, q, k, v)
    need = w.batch * w.n_kv_heads * H.max_granules(run.cfg)
    cache = need + 64  # below the 1024 granules of the 4 (sequence, KV head) slabs
    _, _, cold = run_host_tier(run, max_window_chunks=4, slots=need + 64)
    out, lse, stats = run_host_tier(run, max_window_chunks=4, slots=need + 64, cache_slots=cache)
    print(f"[gpu] warm tier {base}: {stats} (no cache: {cold})", flush=True)
    same = (bool(torch.equal(out, run.out)), bool(torch.equal(lse, run.lse)))
    assert all(same), same
    assert stats["granules_hit"] > 0
    assert stats["granules_copied"] < cold["granules_copied"]
    assert stats["granules_copied"] > cache          # slots were evicted and reused
    assert stats["windows"] >= w.n_q // w.chunk_size // 4


def test_host_tier_same_stream_and_no_threads():
    """Copy and compute on one stream, packing on the calling thread."""
    import torch
    w = W.HOST_TIERED_GROUP.scaled(n_ctx=4096, kv_cap=4096, n_q=4096, planted=8)
    q, k, v = P.make_inputs_parallel(w)
    run = P.DeviceRun(w, q, k, v)
    slots = 2 * w.batch * w.n_kv_heads * H.max_granules(run.cfg)
    out, lse, stats = run_host_tier(run, 8, slots, threads=0, copy_stream=False)
    same = bool(torch.equal(out, run.out))
    assert same


def test_host_tier_rejects_pageable_memory():
    import torch
    w = W.HOST_TIERED_GROUP.scaled(n_ctx=1024, kv_cap=1024, n_q=1024, planted=0)
    q, k, v = P.make_inputs_parallel(w)
    run = P.DeviceRun(w, q, k, v, attend=False)
    cfg = run.cfg
    B, Hkv, cap, d = run.k.shape
    pageable = torch.zeros((B, Hkv, cap // w.group_size, 2, w.group_size, d), dtype=torch.bfloat16)
    slots = B * Hkv * H.max_granules(cfg)
    dev_b, host_b = H.host_tiered_buffer_bytes(cfg, torch.bfloat16, B, 0, w.n_q, 4, slots)
    dev = torch.empty(dev_b, dtype=torch.uint8, device="cuda:0")
    host = torch.empty(host_b, dtype=torch.uint8, pin_memory=True)
    import ctypes
    stats = H.hga_tier_stats()
    st = H.lib().hga_attend_host_tiered(
        ctypes.byref(cfg.c()), H.HGA_BF16, B, run.q.data_ptr(), 0, w.n_q, pageable.data_ptr(), cap,
        run.csum.data_ptr(), run.gsum.data_ptr(), run.out.data_ptr(), None, dev.data_ptr(), dev_b,
        host.data_ptr(), host_b, 4, slots, 0, 2, None, None, ctypes.byref(stats))
    assert st == 1
    # the failed pointer query left no error behind for the next launch
    run.attend()
    torch.cuda.synchronize()


@pytest.mark.parametrize("i", range(0, N_CONFIGS, 2))
def test_host_tier_random_shapes(i):
    """The random parity shapes through the host tier: cold, with random
    window sizes and slot counts, against the oracle; with a warm tier and
    other window and slot sizes, equal to the cold run bit for bit (each
    unit's attention does not depend on its window or on where its granules
    sit in the pool).  The device path is not the reference here: for
    few-unit calls it splits each unit's keys over workgroups, or takes the
    decode kernel for units of at most 16 rows, which the host tier does not,
    so the two agree only to rounding on such shapes."""
    import torch
    w = random_workload(i)
    rng = np.random.default_rng(500 + i)
    q, k, v = P.make_inputs_parallel(w, seed=i)
    run = P.DeviceRun(w, q, k, v)
    need = w.batch * w.n_kv_heads * H.max_granules(run.cfg)
    draws = [(need + int(rng.integers(0, 2 * need + 1)), int(rng.integers(1, 9))) for _ in range(2)]
    cache = need + int(rng.integers(0, need + 1))
    print(f"[gpu] host tier random {i}: {w} (slots, window) {draws} cache {cache}", flush=True)
    out, lse, cold = run_host_tier(run, max_window_chunks=draws[0][1], slots=draws[0][0],
                                   threads=int(rng.integers(0, 4)))
    P.check_attention(run, q, k, v, P.all_units(w), out=out.float().cpu().numpy(), lse=lse.cpu().numpy())
    out2, lse2, warm = run_host_tier(run, max_window_chunks=draws[1][1], slots=draws[1][0],
                                     cache_slots=cache, threads=int(rng.integers(0, 4)))
    same = (bool(torch.equal(out2, out)), bool(torch.equal(lse2, lse)))
    assert all(same), (same, cold, warm)
