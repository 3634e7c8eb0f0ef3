"""MI355X (gfx950) routed exact-token attention -- Hierarchical Global Attention.

A thin ctypes binding over ``libhga.so`` (built from ``csrc/`` by
``python -m hierarchical_kv_routing_amd.build``).  Every step of the path
runs in the library's HIP kernels; this module only checks tensor shapes and
passes device pointers and the current HIP stream.  PyTorch provides device
memory and streams.  There is no fallback: a missing or unloadable library
raises ``HGAError``.

Entry points (same names as the C ABI in include/hga.h):
  build_summaries  -- rotated key cache + mixed-RoPE chunk / group summaries
  route            -- chunk top-K_c, group top-K_g, visible granule lists
  attend           -- exact-token softmax attention over the granule lists
  dense_causal     -- Eq. (1) dense causal attention (reference path)
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhga.so")

HGA_OK = 0
_STATUS = {0: "HGA_OK", 1: "HGA_ERR_INVALID_ARGUMENT", 2: "HGA_ERR_UNSUPPORTED",
           3: "HGA_ERR_WORKSPACE_TOO_SMALL", 4: "HGA_ERR_HIP"}
HGA_F32, HGA_BF16 = 0, 1

# Every symbol include/hga.h declares.
ABI_SYMBOLS = ("hga_build_summaries", "hga_max_granules", "hga_route_workspace_bytes",
               "hga_route", "hga_attend_workspace_bytes", "hga_attend", "hga_dense_causal",
               "hga_host_tiered_buffer_bytes", "hga_host_tiered_cache_slots", "hga_attend_host_tiered",
               "hga_decode_session_cache_slots", "hga_decode_session_buffer_bytes",
               "hga_decode_session_create",
               "hga_decode_session_destroy", "hga_decode_session_append",
               "hga_decode_session_step", "hga_attend_backward_workspace_bytes",
               "hga_attend_backward", "hga_attend_noalloc", "hga_attend_noalloc_max_scratch_bytes",
               "hga_decode_step_workspace_bytes", "hga_decode_step",
               "hga_status_string", "hga_last_hip_error")


class HGAError(RuntimeError):
    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


class hga_config(ctypes.Structure):
    _fields_ = [("chunk_size", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("n_sink_chunks", ctypes.c_int32), ("n_recent_chunks", ctypes.c_int32),
                ("top_chunks", ctypes.c_int32), ("top_groups", ctypes.c_int32),
                ("n_hf_pairs", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("softmax_scale", ctypes.c_float),
                ("rope_period", ctypes.c_int64)]


class hga_tier_stats(ctypes.Structure):
    _fields_ = [("windows", ctypes.c_int64), ("granules_copied", ctypes.c_int64),
                ("bytes_h2d", ctypes.c_int64), ("pack_seconds", ctypes.c_double),
                ("host_seconds", ctypes.c_double), ("granules_hit", ctypes.c_int64)]


@dataclass(frozen=True)
class Config:
    """Routing / attention parameters (names of the pages: C, g_s, F, L, K_c, K_g)."""
    chunk_size: int
    group_size: int
    n_sink_chunks: int
    n_recent_chunks: int
    top_chunks: int
    top_groups: int
    n_hf_pairs: int
    head_dim: int
    n_q_heads: int
    n_kv_heads: int
    rope_theta: float
    softmax_scale: float = 0.0
    rope_period: int = 0  # RoPE positions wrap modulo this (0 = absolute)

    @classmethod
    def from_workload(cls, w, **over) -> "Config":
        kw = dict(chunk_size=w.chunk_size, group_size=w.group_size,
                  n_sink_chunks=w.n_sink_chunks, n_recent_chunks=w.n_recent_chunks,
                  top_chunks=w.top_chunks, top_groups=w.top_groups, n_hf_pairs=w.n_hf_pairs,
                  head_dim=w.head_dim, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                  rope_theta=w.rope_theta, rope_period=w.rope_period)
        kw.update(over)
        return cls(**kw)

    def c(self) -> hga_config:
        return hga_config(self.chunk_size, self.group_size, self.n_sink_chunks,
                          self.n_recent_chunks, self.top_chunks, self.top_groups,
                          self.n_hf_pairs, self.head_dim, self.n_q_heads, self.n_kv_heads,
                          float(self.rope_theta), float(self.softmax_scale),
                          int(self.rope_period))

    def n_query_chunks(self, q_pos0: int, n_q: int) -> int:
        if n_q <= 0:
            return 0
        return (q_pos0 + n_q - 1) // self.chunk_size - q_pos0 // self.chunk_size + 1


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libhga.so (raises HGAError when it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise HGAError(f"{LIB_PATH} is not built; run: python -m hierarchical_kv_routing_amd.build")
    # torch first: its HIP runtime carries the soname the library links
    # against, so the library binds to it.  Loaded the other way round, the
    # process would hold two HIP runtimes, and the library's would find no
    # device once torch's owns it.
    import torch  # noqa: F401
    try:
        l = ctypes.CDLL(LIB_PATH)
    except OSError as e:
        raise HGAError(f"cannot load {LIB_PATH}: {e}") from e
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    CP = ctypes.POINTER(hga_config)
    sig = {
        "hga_build_summaries": (I32, [CP, I32, I32, P, I64, I64, I64, P, P, P, P]),
        "hga_max_granules": (I32, [CP]),
        "hga_route_workspace_bytes": (SZ, [CP, I32, I64, I64]),
        "hga_route": (I32, [CP, I32, I32, P, I64, I64, P, P, I64, P, P, P, P, P, SZ, P]),
        "hga_attend_workspace_bytes": (SZ, [CP, I32, I64, I64]),
        "hga_attend": (I32, [CP, I32, I32, P, I64, I64, P, P, I64, P, P, P, P, P, SZ, P]),
        "hga_dense_causal": (I32, [CP, I32, I32, P, I64, I64, P, P, I64, P, P, P, SZ, P]),
        "hga_attend_noalloc": (I32, [CP, I32, I32, P, I64, I64, P, P, I64, P, P, P, P, P]),
        "hga_attend_noalloc_max_scratch_bytes": (SZ, []),
        "hga_decode_step_workspace_bytes": (SZ, [CP, I32, I64]),
        "hga_decode_step": (I32, [CP, I32, I32, P, I64, P, P, I64, P, P, P, P, P, P, P, P, P, SZ, P]),
        "hga_host_tiered_buffer_bytes": (I32, [CP, I32, I32, I64, I64, I32, I64, I64,
                                               ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
        "hga_host_tiered_cache_slots": (I32, [CP, I32, I32, I64, I64, I32, I64, SZ, ctypes.POINTER(I64)]),
        "hga_decode_session_cache_slots": (I32, [CP, I32, I32, I64, SZ, ctypes.POINTER(I64)]),
        "hga_attend_host_tiered": (I32, [CP, I32, I32, P, I64, I64, P, I64, P, P, P, P, P, SZ, P, SZ,
                                         I32, I64, I64, I32, P, P, ctypes.POINTER(hga_tier_stats)]),
        "hga_decode_session_buffer_bytes": (I32, [CP, I32, I32, I64, I64, ctypes.POINTER(SZ),
                                                  ctypes.POINTER(SZ)]),
        "hga_decode_session_create": (I32, [CP, I32, I32, I64, I64, I64, P, P, SZ, P, SZ,
                                            ctypes.POINTER(P)]),
        "hga_decode_session_destroy": (None, [P]),
        "hga_decode_session_append": (I32, [P, P, P, I64, P, P, P]),
        "hga_decode_session_step": (I32, [P, P, I64, P, P, P, P, P, ctypes.POINTER(hga_tier_stats)]),
        "hga_attend_backward_workspace_bytes": (SZ, [CP, I32, I64, I64]),
        "hga_attend_backward": (I32, [CP, I32, I32, P, I64, I64, P, P, I64, P, P, P, P, P, P, P, P,
                                      P, SZ, P]),
        "hga_status_string": (ctypes.c_char_p, [I32]),
        "hga_last_hip_error": (ctypes.c_int, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(l, name)
        f.restype = res
        f.argtypes = args
    _lib = l
    return _lib


def _check(status: int, what: str):
    if status != HGA_OK:
        extra = ""
        if status == 4:
            extra = f" (hipError {lib().hga_last_hip_error()})"
        raise HGAError(f"{what}: {_STATUS.get(status, status)}{extra}", status)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return HGA_BF16
    if t.dtype == torch.float32:
        return HGA_F32
    raise HGAError(f"unsupported dtype {t.dtype}: q/k/v/out must be bfloat16 or float32")


def _dev(t, name, shape=None, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise HGAError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise HGAError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise HGAError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise HGAError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _stream(t, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def max_granules(cfg: Config) -> int:
    return int(lib().hga_max_granules(ctypes.byref(cfg.c())))


def route_workspace_bytes(cfg: Config, batch: int, q_pos0: int, n_q: int) -> int:
    return int(lib().hga_route_workspace_bytes(ctypes.byref(cfg.c()), batch, q_pos0, n_q))


def attend_workspace_bytes(cfg: Config, batch: int, q_pos0: int, n_q: int) -> int:
    return int(lib().hga_attend_workspace_bytes(ctypes.byref(cfg.c()), batch, q_pos0, n_q))


def build_summaries(cfg: Config, k_raw, tok_begin: int, tok_end: int, k_rot, chunk_sum,
                    group_sum=None, stream=None):
    """Rotate keys [tok_begin, tok_end) into k_rot and write the summaries of
    every chunk / group that closes inside the range (the store's append)."""
    torch = _torch()
    B, Hkv, cap, d = k_raw.shape
    _dev(k_raw, "k_raw")
    _dev(k_rot, "k_rot", k_raw.shape, k_raw.dtype)
    _dev(chunk_sum, "chunk_sum", (B, Hkv, cap // cfg.chunk_size, d), torch.float32)
    _dev(group_sum, "group_sum", (B, Hkv, cap // cfg.group_size, d), torch.float32)
    st = lib().hga_build_summaries(
        ctypes.byref(cfg.c()), _dtype_code(k_raw), B, k_raw.data_ptr(), cap, tok_begin, tok_end,
        k_rot.data_ptr() if k_rot is not None else None, chunk_sum.data_ptr(),
        group_sum.data_ptr() if group_sum is not None else None, _stream(k_raw, stream))
    _check(st, "hga_build_summaries")


def route_outputs(cfg: Config, batch: int, q_pos0: int, n_q: int, device):
    """Allocate chunk_idx, group_idx, granules, granule_count and the workspace."""
    torch = _torch()
    nqc = cfg.n_query_chunks(q_pos0, n_q)
    H = cfg.n_kv_heads
    out = dict(
        chunk_idx=torch.empty((batch, H, nqc, max(cfg.top_chunks, 1)), dtype=torch.int32, device=device),
        group_idx=torch.empty((batch, H, nqc, max(cfg.top_groups, 1)), dtype=torch.int32, device=device),
        granules=torch.empty((batch, H, nqc, max_granules(cfg)), dtype=torch.int32, device=device),
        granule_count=torch.empty((batch, H, nqc), dtype=torch.int32, device=device))
    ws = route_workspace_bytes(cfg, batch, q_pos0, n_q)
    out["workspace"] = torch.empty(max(ws, 16), dtype=torch.uint8, device=device)
    return out


def route(cfg: Config, q, q_pos0: int, chunk_sum, group_sum, kv_cap: int, chunk_idx, group_idx,
          granules, granule_count, workspace=None, stream=None):
    """Two-level routing of every (sequence, KV head, query chunk) unit."""
    torch = _torch()
    B, Hq, n_q, d = q.shape
    nqc = cfg.n_query_chunks(q_pos0, n_q)
    Hkv = cfg.n_kv_heads
    _dev(q, "q")
    _dev(chunk_sum, "chunk_sum", (B, Hkv, kv_cap // cfg.chunk_size, d), torch.float32)
    _dev(group_sum, "group_sum", (B, Hkv, kv_cap // cfg.group_size, d), torch.float32)
    _dev(chunk_idx, "chunk_idx", (B, Hkv, nqc, max(cfg.top_chunks, 1)), torch.int32)
    _dev(group_idx, "group_idx", (B, Hkv, nqc, max(cfg.top_groups, 1)), torch.int32)
    _dev(granules, "granules", (B, Hkv, nqc, max_granules(cfg)), torch.int32)
    _dev(granule_count, "granule_count", (B, Hkv, nqc), torch.int32)
    _dev(workspace, "workspace")
    st = lib().hga_route(
        ctypes.byref(cfg.c()), _dtype_code(q), B, q.data_ptr(), q_pos0, n_q,
        chunk_sum.data_ptr(), group_sum.data_ptr() if group_sum is not None else None, kv_cap,
        chunk_idx.data_ptr(), group_idx.data_ptr() if group_idx is not None else None,
        granules.data_ptr(), granule_count.data_ptr(),
        workspace.data_ptr() if workspace is not None else None,
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(q, stream))
    _check(st, "hga_route")


def attend(cfg: Config, q, q_pos0: int, k_rot, v, granules, granule_count, out, lse=None,
           workspace=None, stream=None):
    """Exact-token attention of every query over its unit's granule list."""
    torch = _torch()
    B, Hq, n_q, d = q.shape
    kv_cap = k_rot.shape[2]
    nqc = cfg.n_query_chunks(q_pos0, n_q)
    _dev(q, "q")
    _dev(k_rot, "k_rot", (B, cfg.n_kv_heads, kv_cap, d), q.dtype)
    _dev(v, "v", (B, cfg.n_kv_heads, kv_cap, d), q.dtype)
    _dev(granules, "granules", (B, cfg.n_kv_heads, nqc, max_granules(cfg)), torch.int32)
    _dev(granule_count, "granule_count", (B, cfg.n_kv_heads, nqc), torch.int32)
    _dev(out, "out", q.shape, q.dtype)
    _dev(lse, "lse", (B, Hq, n_q), torch.float32)
    _dev(workspace, "workspace")
    st = lib().hga_attend(
        ctypes.byref(cfg.c()), _dtype_code(q), B, q.data_ptr(), q_pos0, n_q, k_rot.data_ptr(),
        v.data_ptr(), kv_cap, granules.data_ptr(), granule_count.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None,
        workspace.data_ptr() if workspace is not None else None,
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(q, stream))
    _check(st, "hga_attend")


def attend_noalloc(cfg: Config, q, q_pos0: int, k_rot, v, granules, granule_count, out, lse=None,
                   stream=None):
    """hga_attend with the library's static device scratch instead of a
    workspace (allocates nothing; calls on one device must not overlap)."""
    torch = _torch()
    B, Hq, n_q, d = q.shape
    kv_cap = k_rot.shape[2]
    nqc = cfg.n_query_chunks(q_pos0, n_q)
    _dev(q, "q")
    _dev(k_rot, "k_rot", (B, cfg.n_kv_heads, kv_cap, d), q.dtype)
    _dev(v, "v", (B, cfg.n_kv_heads, kv_cap, d), q.dtype)
    _dev(granules, "granules", (B, cfg.n_kv_heads, nqc, max_granules(cfg)), torch.int32)
    _dev(granule_count, "granule_count", (B, cfg.n_kv_heads, nqc), torch.int32)
    _dev(out, "out", q.shape, q.dtype)
    _dev(lse, "lse", (B, Hq, n_q), torch.float32)
    st = lib().hga_attend_noalloc(
        ctypes.byref(cfg.c()), _dtype_code(q), B, q.data_ptr(), q_pos0, n_q, k_rot.data_ptr(),
        v.data_ptr(), kv_cap, granules.data_ptr(), granule_count.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, _stream(q, stream))
    _check(st, "hga_attend_noalloc")


def attend_noalloc_max_scratch_bytes() -> int:
    return int(lib().hga_attend_noalloc_max_scratch_bytes())


def decode_step_workspace_bytes(cfg: Config, batch: int, pos: int) -> int:
    return int(lib().hga_decode_step_workspace_bytes(ctypes.byref(cfg.c()), batch, pos))


def decode_step_workspace(cfg: Config, batch: int, pos: int, device):
    """A workspace for hga_decode_step (no initial contents needed)."""
    torch = _torch()
    n = decode_step_workspace_bytes(cfg, batch, pos)
    if n == 0:
        raise HGAError("hga_decode_step does not support this shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def decode_step(cfg: Config, q, pos: int, k_rot, v, chunk_sum, group_sum, out, lse=None,
                lists=None, workspace=None, stream=None):
    """One decode step (query of every sequence at position pos) in two
    launches: routing, gather and attention.  ``lists`` (optional): dict with
    chunk_idx, group_idx, granules, granule_count as route_outputs(cfg, B,
    pos, 1) allocates them."""
    torch = _torch()
    B, Hq, n_q, d = q.shape
    if n_q != 1:
        raise HGAError("decode_step takes one query per sequence")
    kv_cap = k_rot.shape[2]
    Hkv = cfg.n_kv_heads
    _dev(q, "q")
    _dev(k_rot, "k_rot", (B, Hkv, kv_cap, d), q.dtype)
    _dev(v, "v", (B, Hkv, kv_cap, d), q.dtype)
    _dev(chunk_sum, "chunk_sum", (B, Hkv, kv_cap // cfg.chunk_size, d), torch.float32)
    _dev(group_sum, "group_sum", (B, Hkv, kv_cap // cfg.group_size, d), torch.float32)
    _dev(out, "out", q.shape, q.dtype)
    _dev(lse, "lse", (B, Hq, 1), torch.float32)
    _dev(workspace, "workspace")
    ptr = lambda name: lists[name].data_ptr() if lists is not None else None  # noqa: E731
    if lists is not None:
        _dev(lists["chunk_idx"], "chunk_idx", (B, Hkv, 1, max(cfg.top_chunks, 1)), torch.int32)
        _dev(lists["group_idx"], "group_idx", (B, Hkv, 1, max(cfg.top_groups, 1)), torch.int32)
        _dev(lists["granules"], "granules", (B, Hkv, 1, max_granules(cfg)), torch.int32)
        _dev(lists["granule_count"], "granule_count", (B, Hkv, 1), torch.int32)
    st = lib().hga_decode_step(
        ctypes.byref(cfg.c()), _dtype_code(q), B, q.data_ptr(), pos, k_rot.data_ptr(), v.data_ptr(),
        kv_cap, chunk_sum.data_ptr(), group_sum.data_ptr() if group_sum is not None else None,
        ptr("chunk_idx"), ptr("group_idx"), ptr("granules"), ptr("granule_count"),
        out.data_ptr(), lse.data_ptr() if lse is not None else None,
        workspace.data_ptr() if workspace is not None else None,
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(q, stream))
    _check(st, "hga_decode_step")


def dense_causal(cfg: Config, q, q_pos0: int, k_rot, v, out, lse=None, workspace=None, stream=None):
    """Eq. (1): every query attends to all keys at positions <= its own."""
    torch = _torch()
    B, Hq, n_q, d = q.shape
    kv_cap = k_rot.shape[2]
    _dev(q, "q")
    _dev(k_rot, "k_rot", (B, cfg.n_kv_heads, kv_cap, d), q.dtype)
    _dev(v, "v", (B, cfg.n_kv_heads, kv_cap, d), q.dtype)
    _dev(out, "out", q.shape, q.dtype)
    _dev(lse, "lse", (B, Hq, n_q), torch.float32)
    _dev(workspace, "workspace")
    st = lib().hga_dense_causal(
        ctypes.byref(cfg.c()), _dtype_code(q), B, q.data_ptr(), q_pos0, n_q, k_rot.data_ptr(),
        v.data_ptr(), kv_cap, out.data_ptr(), lse.data_ptr() if lse is not None else None,
        workspace.data_ptr() if workspace is not None else None,
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(q, stream))
    _check(st, "hga_dense_causal")


def host_tiered_buffer_bytes(cfg: Config, dtype, batch: int, q_pos0: int, n_q: int,
                             max_window_chunks: int, slots_per_window: int, cache_slots: int = 0):
    """(device_bytes, host_bytes) of the staging buffers the host tier needs
    (cache_slots > 0: with a warm tier of that many granules)."""
    torch = _torch()
    code = HGA_BF16 if dtype == torch.bfloat16 else HGA_F32
    dev, host = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = lib().hga_host_tiered_buffer_bytes(ctypes.byref(cfg.c()), code, batch, q_pos0, n_q,
                                            max_window_chunks, slots_per_window, cache_slots,
                                            ctypes.byref(dev), ctypes.byref(host))
    _check(st, "hga_host_tiered_buffer_bytes")
    return dev.value, host.value


def host_tiered_cache_slots(cfg: Config, dtype, batch: int, q_pos0: int, n_q: int,
                            max_window_chunks: int, slots_per_window: int, headroom_bytes: int) -> int:
    """Warm-tier granules that fit while headroom_bytes of the device's free
    memory stay unused (0: the cold tier alone)."""
    torch = _torch()
    code = HGA_BF16 if dtype == torch.bfloat16 else HGA_F32
    n = ctypes.c_int64(0)
    st = lib().hga_host_tiered_cache_slots(ctypes.byref(cfg.c()), code, batch, q_pos0, n_q,
                                           max_window_chunks, slots_per_window, headroom_bytes,
                                           ctypes.byref(n))
    _check(st, "hga_host_tiered_cache_slots")
    return n.value


def decode_session_cache_slots(cfg: Config, dtype, batch: int, kv_cap: int, headroom_bytes: int) -> int:
    """Decode-session cache granules that fit while headroom_bytes of the
    device's free memory stay unused."""
    torch = _torch()
    code = HGA_BF16 if dtype == torch.bfloat16 else HGA_F32
    n = ctypes.c_int64(0)
    st = lib().hga_decode_session_cache_slots(ctypes.byref(cfg.c()), code, batch, kv_cap, headroom_bytes,
                                              ctypes.byref(n))
    _check(st, "hga_decode_session_cache_slots")
    return n.value


def host_store(cfg: Config, k_rot, v):
    """Pinned host copy of (rotated K, V) in the granule-major layout the host
    tier reads: [B][Hkv][kv_cap/g_s][2][g_s][d]."""
    torch = _torch()
    B, Hkv, cap, d = k_rot.shape
    gs = cfg.group_size
    ng = cap // gs
    store = torch.empty((B, Hkv, ng, 2, gs, d), dtype=k_rot.dtype, pin_memory=True)
    both = torch.stack([k_rot.view(B, Hkv, ng, gs, d), v.view(B, Hkv, ng, gs, d)], dim=3)
    store.copy_(both)
    return store


def attend_host_tiered(cfg: Config, q, q_pos0: int, kv_host, kv_cap: int, chunk_sum, group_sum,
                       out, lse, dev_staging, host_staging, max_window_chunks: int,
                       slots_per_window: int, n_threads: int = 8, compute_stream=None,
                       copy_stream=None, cache_slots: int = 0) -> dict:
    """Route + attention with token K/V in pinned host RAM (host-blocking until
    the last attention launch is enqueued), with a warm tier of cache_slots
    granules when cache_slots > 0.  Returns the call's statistics."""
    torch = _torch()
    B, Hq, n_q, d = q.shape
    _dev(q, "q")
    _dev(out, "out", q.shape, q.dtype)
    _dev(lse, "lse", (B, Hq, n_q), torch.float32)
    _dev(chunk_sum, "chunk_sum", (B, cfg.n_kv_heads, kv_cap // cfg.chunk_size, d), torch.float32)
    _dev(group_sum, "group_sum", (B, cfg.n_kv_heads, kv_cap // cfg.group_size, d), torch.float32)
    _dev(dev_staging, "dev_staging")
    if kv_host.is_cuda or not kv_host.is_pinned() or not host_staging.is_pinned():
        raise HGAError("kv_host and host_staging must be pinned host tensors")
    if tuple(kv_host.shape) != (B, cfg.n_kv_heads, kv_cap // cfg.group_size, 2, cfg.group_size, d):
        raise HGAError(f"kv_host has shape {tuple(kv_host.shape)}")
    cs = compute_stream if compute_stream is not None else torch.cuda.current_stream(q.device)
    xs = copy_stream if copy_stream is not None else cs
    stats = hga_tier_stats()
    st = lib().hga_attend_host_tiered(
        ctypes.byref(cfg.c()), _dtype_code(q), B, q.data_ptr(), q_pos0, n_q, kv_host.data_ptr(),
        kv_cap, chunk_sum.data_ptr(), group_sum.data_ptr() if group_sum is not None else None,
        out.data_ptr(), lse.data_ptr() if lse is not None else None,
        dev_staging.data_ptr(), dev_staging.numel() * dev_staging.element_size(),
        host_staging.data_ptr(), host_staging.numel() * host_staging.element_size(),
        max_window_chunks, slots_per_window, cache_slots, n_threads, ctypes.c_void_p(cs.cuda_stream),
        ctypes.c_void_p(xs.cuda_stream), ctypes.byref(stats))
    _check(st, "hga_attend_host_tiered")
    return {f: getattr(stats, f) for f, _ in hga_tier_stats._fields_}


def attend_backward_workspace_bytes(cfg: Config, batch: int, q_pos0: int, n_q: int) -> int:
    return int(lib().hga_attend_backward_workspace_bytes(ctypes.byref(cfg.c()), batch, q_pos0, n_q))


def attend_backward(cfg: Config, q, q_pos0: int, k_rot, v, granules, granule_count, out, lse, d_out,
                    dq, dk, dv, workspace, stream=None):
    """dq, dk, dv (f32) of exact-token attention over fixed granule lists."""
    torch = _torch()
    B, Hq, n_q, d = q.shape
    kv_cap = k_rot.shape[2]
    _dev(q, "q")
    for t, name in ((out, "out"), (d_out, "d_out")):
        _dev(t, name, q.shape, q.dtype)
    _dev(lse, "lse", (B, Hq, n_q), torch.float32)
    _dev(k_rot, "k_rot", k_rot.shape, q.dtype)
    _dev(v, "v", k_rot.shape, q.dtype)
    _dev(dq, "dq", q.shape, torch.float32)
    _dev(dk, "dk", k_rot.shape, torch.float32)
    _dev(dv, "dv", k_rot.shape, torch.float32)
    _dev(granules, "granules")
    _dev(granule_count, "granule_count")
    _dev(workspace, "workspace")
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    st = lib().hga_attend_backward(
        ctypes.byref(cfg.c()), _dtype_code(q), B, q.data_ptr(), q_pos0, n_q, k_rot.data_ptr(), v.data_ptr(),
        kv_cap, granules.data_ptr(), granule_count.data_ptr(), out.data_ptr(), lse.data_ptr(),
        d_out.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), ctypes.c_void_p(s.cuda_stream))
    _check(st, "hga_attend_backward")


def decode_session_buffer_bytes(cfg: Config, dtype, batch: int, kv_cap: int, cache_slots: int):
    """(device_bytes, host_bytes) of a streaming decode session's buffers."""
    torch = _torch()
    code = HGA_BF16 if dtype == torch.bfloat16 else HGA_F32
    dev, host = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = lib().hga_decode_session_buffer_bytes(ctypes.byref(cfg.c()), code, batch, kv_cap, cache_slots,
                                               ctypes.byref(dev), ctypes.byref(host))
    _check(st, "hga_decode_session_buffer_bytes")
    return dev.value, host.value


class DecodeSession:
    """Streaming decode from the host tier: K/V history in the pinned
    granule-major store (host_store layout), a device cache of cache_slots
    granules kept across steps.  The session allocates its device and pinned
    host buffers with torch; the store and summary tables belong to the
    caller."""

    def __init__(self, cfg: Config, batch: int, kv_cap: int, first_pos: int, cache_slots: int,
                 kv_host, device="cuda:0"):
        torch = _torch()
        if kv_host.is_cuda or not kv_host.is_pinned():
            raise HGAError("kv_host must be a pinned host tensor")
        d = cfg.head_dim
        if tuple(kv_host.shape) != (batch, cfg.n_kv_heads, kv_cap // cfg.group_size, 2, cfg.group_size, d):
            raise HGAError(f"kv_host has shape {tuple(kv_host.shape)}")
        self.cfg, self.batch, self.kv_cap = cfg, batch, kv_cap
        self._c = cfg.c()
        dev_b, host_b = decode_session_buffer_bytes(cfg, kv_host.dtype, batch, kv_cap, cache_slots)
        self.dev = torch.empty(max(dev_b, 256), dtype=torch.uint8, device=device)
        self.host = torch.empty(max(host_b, 256), dtype=torch.uint8, pin_memory=True)
        self.store = kv_host
        h = ctypes.c_void_p(None)
        st = lib().hga_decode_session_create(
            ctypes.byref(self._c), _dtype_code(kv_host), batch, kv_cap, first_pos, cache_slots,
            kv_host.data_ptr(), self.dev.data_ptr(), self.dev.numel(), self.host.data_ptr(),
            self.host.numel(), ctypes.byref(h))
        _check(st, "hga_decode_session_create")
        self._h = h

    def append(self, k_raw_new, v_new, pos: int, chunk_sum, group_sum, stream=None):
        """Token pos of every sequence: k_raw_new / v_new [B][Hkv][1][d]."""
        torch = _torch()
        cfg = self.cfg
        shape = (self.batch, cfg.n_kv_heads, 1, cfg.head_dim)
        _dev(k_raw_new, "k_raw_new", shape, self.store.dtype)
        _dev(v_new, "v_new", shape, self.store.dtype)
        _dev(chunk_sum, "chunk_sum")
        _dev(group_sum, "group_sum")
        s = stream if stream is not None else torch.cuda.current_stream(k_raw_new.device)
        st = lib().hga_decode_session_append(
            self._h, k_raw_new.data_ptr(), v_new.data_ptr(), pos, chunk_sum.data_ptr(),
            group_sum.data_ptr() if group_sum is not None else None, ctypes.c_void_p(s.cuda_stream))
        _check(st, "hga_decode_session_append")

    def step(self, q, pos: int, chunk_sum, group_sum, out, lse=None, stream=None, stats=True):
        """One query per sequence at position pos: q, out [B][Hq][1][d].
        With stats, waits for the step and returns its cache counts;
        without, only enqueues it and returns None."""
        torch = _torch()
        cfg = self.cfg
        shape = (self.batch, cfg.n_q_heads, 1, cfg.head_dim)
        _dev(q, "q", shape, self.store.dtype)
        _dev(out, "out", shape, self.store.dtype)
        _dev(lse, "lse", shape[:3], torch.float32)
        _dev(chunk_sum, "chunk_sum")
        _dev(group_sum, "group_sum")
        cs = stream if stream is not None else torch.cuda.current_stream(q.device)
        rec = hga_tier_stats() if stats else None
        st = lib().hga_decode_session_step(
            self._h, q.data_ptr(), pos, chunk_sum.data_ptr(),
            group_sum.data_ptr() if group_sum is not None else None, out.data_ptr(),
            lse.data_ptr() if lse is not None else None, ctypes.c_void_p(cs.cuda_stream),
            ctypes.byref(rec) if rec is not None else None)
        _check(st, "hga_decode_session_step")
        if rec is None:
            return None
        return {f: getattr(rec, f) for f, _ in hga_tier_stats._fields_}

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value is not None:
            lib().hga_decode_session_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def default_scale(cfg: Config) -> float:
    return cfg.softmax_scale if cfg.softmax_scale else 1.0 / math.sqrt(cfg.head_dim)
