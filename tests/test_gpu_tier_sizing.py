"""GPU tests of the warm-tier sizing under a VRAM headroom
(hga_host_tiered_cache_slots, hga_decode_session_cache_slots): the returned
size is the largest whose staging leaves the headroom of the device's free
memory unused, 0 (cold tier) or an error when nothing fits, capped at one
slot per granule; a call with the returned size equals the device path."""
import pytest

import hierarchical_kv_routing_amd as H
import workloads as W
from tests import parity as P
from tests.test_gpu_host_tier import run_host_tier

pytestmark = pytest.mark.gpu


def _tier_case():
    w = W.HOST_TIERED_GROUP.scaled(n_ctx=4096, kv_cap=4096, n_q=4096, planted=16)
    cfg = H.Config.from_workload(w)
    slots = w.batch * w.n_kv_heads * H.max_granules(cfg) + 64
    return w, cfg, slots


def test_host_tier_cache_slots_fit_the_headroom():
    import torch
    w, cfg, slots = _tier_case()
    dt = P.torch_dtype(w)
    lo = w.batch * w.n_kv_heads * H.max_granules(cfg)
    hi = w.batch * w.n_kv_heads * (w.kv_cap // w.group_size)
    need = lambda n: H.host_tiered_buffer_bytes(cfg, dt, w.batch, w.q_pos0, w.n_q, 16, slots, n)[0]
    free = torch.cuda.mem_get_info()[0]
    # room for the smallest tier plus ~10 granules beyond it
    gb = 2 * w.group_size * w.head_dim * 2
    headroom = free - need(lo) - 10 * gb - gb // 2
    n = H.host_tiered_cache_slots(cfg, dt, w.batch, w.q_pos0, w.n_q, 16, slots, headroom)
    budget = torch.cuda.mem_get_info()[0] - headroom
    print(f"[gpu] tier sizing: lo {lo} hi {hi} -> {n}", flush=True)
    assert lo <= n < hi and need(n) <= budget < need(n + 1)
    # no room: the cold tier; no headroom: every granule of the context
    assert H.host_tiered_cache_slots(cfg, dt, w.batch, w.q_pos0, w.n_q, 16, slots, free + (1 << 30)) == 0
    assert H.host_tiered_cache_slots(cfg, dt, w.batch, w.q_pos0, w.n_q, 16, slots, 0) == hi


def test_host_tier_with_sized_warm_tier_equals_device_path():
    import torch
    w, cfg, slots = _tier_case()
    q, k, v = P.make_inputs_parallel(w)
    run = P.DeviceRun(w, q, k, v)
    dt = P.torch_dtype(w)
    lo = w.batch * w.n_kv_heads * H.max_granules(cfg)
    gb = 2 * w.group_size * w.head_dim * 2
    need = H.host_tiered_buffer_bytes(cfg, dt, w.batch, w.q_pos0, w.n_q, 16, slots, lo + 300)[0]
    headroom = torch.cuda.mem_get_info()[0] - need - gb // 2
    n = H.host_tiered_cache_slots(cfg, dt, w.batch, w.q_pos0, w.n_q, 16, slots, headroom)
    assert lo <= n
    out, lse, stats = run_host_tier(run, max_window_chunks=16, slots=slots, cache_slots=n)
    print(f"[gpu] sized warm tier ({n} slots): {stats}", flush=True)
    assert stats["granules_hit"] > 0
    assert torch.equal(out, run.out) and torch.equal(lse, run.lse)


def test_decode_session_cache_slots_fit_the_headroom():
    import torch
    w = W.DECODE_64K.scaled(batch=2, n_ctx=8193, kv_cap=8256, q_pos0=8192)
    cfg = H.Config.from_workload(w)
    dt = torch.bfloat16
    lo = w.batch * w.n_kv_heads * H.max_granules(cfg)
    hi = w.batch * w.n_kv_heads * (w.kv_cap // w.group_size)
    need = lambda n: H.decode_session_buffer_bytes(cfg, dt, w.batch, w.kv_cap, n)[0]
    gb = 2 * w.group_size * w.head_dim * 2
    free = torch.cuda.mem_get_info()[0]
    headroom = free - need(lo) - 20 * gb - gb // 2
    n = H.decode_session_cache_slots(cfg, dt, w.batch, w.kv_cap, headroom)
    budget = torch.cuda.mem_get_info()[0] - headroom
    assert lo <= n < hi and need(n) <= budget < need(n + 1)
    assert H.decode_session_cache_slots(cfg, dt, w.batch, w.kv_cap, 0) == hi
    with pytest.raises(H.HGAError):
        H.decode_session_cache_slots(cfg, dt, w.batch, w.kv_cap, free + (1 << 30))
