"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/hga.h declares, and rejects bad arguments on the host before any
HIP call (nothing is enqueued on an error)."""
import ctypes
import os
import re

import pytest

import hierarchical_kv_routing_amd as H
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(H.LIB_PATH):
        pytest.skip("libhga.so not built (python -m hierarchical_kv_routing_amd.build)")
    return H.lib()


def _declared():
    text = open(os.path.join(ROOT, "include", "hga.h")).read()
    return sorted(set(re.findall(r"\b(hga_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported(lib):
    names = _declared()
    assert set(names) == set(H.ABI_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layouts_match_header(tmp_path):
    """The ctypes mirrors of hga_config and hga_tier_stats have the C
    compiler's size and field offsets for include/hga.h."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    fields = {"hga_config": [f for f, _ in H.hga_config._fields_],
              "hga_tier_stats": [f for f, _ in H.hga_tier_stats._fields_]}
    lines = []
    for st, names in fields.items():
        lines.append(f'  printf("%zu\\n", sizeof({st}));')
        lines += [f'  printf("%zu\\n", offsetof({st}, {n}));' for n in names]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdint.h>\n#include <stdio.h>\n'
                   '#include "hga.h"\nint main(void) {\n' + "\n".join(lines) + "\n  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    want = []
    for cls in (H.hga_config, H.hga_tier_stats):
        want.append(ctypes.sizeof(cls))
        want += [getattr(cls, f).offset for f, _ in cls._fields_]
    assert got == want


def test_decode_session_sizes_and_checks(lib):
    """Streaming decode sessions: buffer sizes, and argument checks that fail
    before any HIP call (pointers here are never dereferenced)."""
    cfg = H.Config.from_workload(W.DECODE_64K)
    c = ctypes.byref(cfg.c())
    cap = 65600
    need = 16 * 4 * H.max_granules(cfg)
    dev, host = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.hga_decode_session_buffer_bytes(c, 1, 16, cap, need, ctypes.byref(dev), ctypes.byref(host)) == 0
    granule = 2 * 16 * 128 * 2
    assert dev.value > need * granule and host.value > 0
    # the cache must hold one step's granules; bf16 only
    assert lib.hga_decode_session_buffer_bytes(c, 1, 16, cap, need - 1, ctypes.byref(dev), ctypes.byref(host)) == 1
    assert lib.hga_decode_session_buffer_bytes(c, 0, 16, cap, need, ctypes.byref(dev), ctypes.byref(host)) == 2
    h = ctypes.c_void_p(None)
    # missing buffers, then a first position off a chunk boundary
    assert lib.hga_decode_session_create(c, 1, 16, cap, 65536, need, None, 256, 1 << 30, 256, 1 << 20,
                                         ctypes.byref(h)) == 1
    assert lib.hga_decode_session_create(c, 1, 16, cap, 65537, need, 256, 256, 1 << 30, 256, 1 << 20,
                                         ctypes.byref(h)) == 1
    assert h.value is None
    assert lib.hga_decode_session_append(None, 16, 16, 0, 16, 16, None) == 1
    assert lib.hga_decode_session_step(None, 16, 0, 16, 16, 16, None, None, None) == 1
    lib.hga_decode_session_destroy(None)


def test_backward_checks(lib):
    """hga_attend_backward: workspace size and host-side argument checks."""
    cfg = H.Config.from_workload(W.QWEN3_PREFILL)
    c = ctypes.byref(cfg.c())
    need = H.attend_backward_workspace_bytes(cfg, 1, 0, 32768)
    assert need >= 32 * 32768 * 4
    args = [c, 1, 1, 16, 0, 64, 16, 16, 64, 16, 16, 16, 16, 16, 16, 16, 16, 16, 1 << 20, None]
    bad = list(args)
    bad[3] = None  # no queries
    assert lib.hga_attend_backward(*bad) == 1
    f32 = list(args)
    f32[1] = 0  # f32 inputs: not supported by the backward
    assert lib.hga_attend_backward(*f32) == 2
    small = list(args)
    small[17], small[18] = 16, 4  # workspace too small
    assert lib.hga_attend_backward(*small) == 3


def test_status_strings(lib):
    for code, name in H._STATUS.items():
        assert lib.hga_status_string(code).decode() == name
    assert lib.hga_last_hip_error() == 0


def test_max_granules(lib):
    # (C/g_s)(1 + F + max(L,1)) + routed
    assert H.max_granules(H.Config.from_workload(W.QWEN3_PREFILL)) == 4 * 11 + 32
    assert H.max_granules(H.Config.from_workload(W.HOST_TIERED_CHUNK)) == 4 * 11 + 24 * 4
    assert H.max_granules(H.Config.from_workload(W.TINY_F32)) == 4 * 5 + 4
    assert H.max_granules(H.Config.from_workload(W.TINY_F32, n_recent_chunks=0)) == 4 * 4 + 4
    assert H.max_granules(H.Config.from_workload(W.TINY_F32, group_size=48)) == -1


def _route(lib, cfg, dtype=1, B=1, q=16, q_pos0=0, n_q=64, cs=16, gs=16, cap=64,
           ci=16, gi=16, gr=16, gc=16, ws=None, wsb=0):
    return lib.hga_route(ctypes.byref(cfg.c()), dtype, B, q, q_pos0, n_q, cs, gs, cap, ci, gi, gr, gc,
                         ws, wsb, None)


@pytest.mark.parametrize("over,status", [
    (dict(group_size=48), 1),          # C % g_s != 0
    (dict(group_size=0), 1),
    (dict(n_q_heads=6, n_kv_heads=4), 1),
    (dict(n_hf_pairs=65), 1),
    (dict(n_hf_pairs=-1), 1),
    (dict(top_chunks=-1), 1),
    (dict(rope_theta=0.0), 1),
    (dict(rope_theta=float("nan")), 1),
    (dict(softmax_scale=-1.0), 1),
    (dict(rope_period=-64), 1),
    (dict(rope_period=100), 1),        # wrap period not a multiple of C
    (dict(head_dim=96), 2),            # d in {64, 128}
    (dict(chunk_size=128, group_size=16), 2),
])
def test_bad_config_rejected(lib, over, status):
    cfg = H.Config.from_workload(W.QWEN3_PREFILL, **over)
    # Pointers here are never dereferenced: validation fails first.
    assert _route(lib, cfg) == status
    assert lib.hga_build_summaries(ctypes.byref(cfg.c()), 1, 1, 16, 64, 0, 64, None, 16, 16, None) == status
    assert lib.hga_attend(ctypes.byref(cfg.c()), 1, 1, 16, 0, 64, 16, 16, 64, 16, 16, 16, None,
                          None, 0, None) == status


@pytest.mark.parametrize("over,call", [
    (dict(top_chunks=257), {}),                       # K_c <= 256
    (dict(top_groups=257), {}),                       # K_g <= 256
    (dict(n_q_heads=64, n_kv_heads=4), {}),           # C * G = 1024 rows > 512 per unit
    (dict(top_chunks=256, group_size=2), {}),         # K_c * C / g_s = 8192 candidate groups > 4096
    ({}, dict(q_pos0=4200 * 64, n_q=64, cap=4201 * 64)),  # 4189 middle chunks > 4096
])
def test_route_limits_rejected(lib, over, call):
    """The shape limits hga_route documents in include/hga.h return
    HGA_ERR_UNSUPPORTED before anything is read or launched."""
    cfg = H.Config.from_workload(W.QWEN3_PREFILL, **over)
    assert _route(lib, cfg, **call) == 2


@pytest.mark.parametrize("over,cap,dtype,status", [
    (dict(chunk_size=48, group_size=12), 4800, 1, 2),   # g_s not a power of two
    ({}, 1 << 23, 1, 2),                               # bf16 slab kv_cap * d * 2 = 2^31 bytes
    ({}, (1 << 23) - 64, 1, "ok"),                     # just below: accepted by the size rule
    ({}, 1 << 23, 0, "ok"),                            # f32 slabs are not buffer-addressed
])
def test_attend_limits_rejected(lib, over, cap, dtype, status):
    """hga_attend's documented limits: g_s a power of two, bf16 (sequence, KV
    head) slabs below 2^31 bytes.  Accepted shapes fail later, on the null
    output pointer (HGA_ERR_INVALID_ARGUMENT); nothing is ever launched."""
    cfg = H.Config.from_workload(W.QWEN3_PREFILL, **over)
    rc = lib.hga_attend(ctypes.byref(cfg.c()), dtype, 1, 16, 0, 64, 16, 16, cap, 16, 16, None, None,
                        None, 0, None)
    assert rc == (1 if status == "ok" else status)


def test_bad_arguments_rejected(lib):
    cfg = H.Config.from_workload(W.QWEN3_PREFILL)
    assert _route(lib, cfg, dtype=7) == 1
    assert _route(lib, cfg, B=0) == 1
    assert _route(lib, cfg, cap=100) == 1              # kv_cap % C
    assert _route(lib, cfg, n_q=65) == 1               # q_pos0 + n_q > kv_cap
    assert _route(lib, cfg, q_pos0=-1) == 1
    assert _route(lib, cfg, q=None) == 1
    assert _route(lib, cfg, q=18) == 1                 # misaligned
    assert _route(lib, cfg, gr=None) == 1
    assert _route(lib, cfg, gs=None) == 1              # K_g > 0 needs group summaries
    assert _route(lib, cfg, n_q=0) == 0                # empty call: a no-op
    # summaries: empty / reversed / out-of-range token ranges
    c = ctypes.byref(cfg.c())
    assert lib.hga_build_summaries(c, 1, 1, 16, 64, 10, 10, None, 16, 16, None) == 1
    assert lib.hga_build_summaries(c, 1, 1, 16, 64, 0, 65, None, 16, 16, None) == 1
    assert lib.hga_build_summaries(c, 1, 1, 16, 64, 0, 64, None, 16, None, None) == 1
    # dense / attend null pointers
    assert lib.hga_dense_causal(c, 1, 1, 16, 0, 64, None, 16, 64, 16, None, None, 0, None) == 1
    assert lib.hga_attend(c, 1, 1, 16, 0, 64, 16, 16, 64, None, 16, 16, None, None, 0, None) == 1


def test_workspace_checks(lib):
    cfg = H.Config.from_workload(W.DECODE_64K)
    # 4 sequences x 4 KV heads = 16 units: segmented decode routing over 1014
    # middle chunks, 16 segments of 64 chunks, each keeping its top K_c = 8
    # (a key and a chunk offset) and the scores of their 4 groups each, all
    # 4-byte words
    need = H.route_workspace_bytes(cfg, 4, 65536, 1)
    assert need == 4 * 4 * 16 * 8 * (2 + 4) * 4
    assert _route(lib, cfg, B=4, q_pos0=65536, n_q=1, cap=65600, ws=16, wsb=need - 4) == 3
    assert _route(lib, cfg, B=4, q_pos0=65536, n_q=1, cap=65600, ws=None, wsb=0) == 3
    # 64 units: 8 segments of 128 chunks
    assert H.route_workspace_bytes(cfg, 16, 65536, 1) == 16 * 4 * 8 * 8 * (2 + 4) * 4
    # chunk routing only: no group keys
    chunk_only = H.Config.from_workload(W.DECODE_64K, top_groups=0)
    assert H.route_workspace_bytes(chunk_only, 16, 65536, 1) == 16 * 4 * 8 * 8 * 2 * 4
    assert H.attend_workspace_bytes(cfg, 16, 65536, 1) > 0
    # no routing (K_c = 0): nothing to keep
    assert H.route_workspace_bytes(H.Config.from_workload(W.DECODE_64K, top_chunks=0), 16, 65536, 1) == 0
    # many query chunks: one routing workgroup per unit
    big = H.Config.from_workload(W.QWEN3_PREFILL)
    # prefill: the summary tables split into bf16 hi / lo rows for the staged
    # scoring, then the norms of the chunk rows (f32) for the screening bound
    assert H.route_workspace_bytes(big, 1, 0, 32768) == 4 * (512 + 512 * 4) * 128 * 2 * 2 + 4 * 512 * 4


def test_host_tier_sizes_and_checks(lib):
    cfg = H.Config.from_workload(W.HOST_TIERED_GROUP)
    gmax = H.max_granules(cfg)
    dev, host = ctypes.c_size_t(0), ctypes.c_size_t(0)
    c = ctypes.byref(cfg.c())
    assert lib.hga_host_tiered_buffer_bytes(c, 1, 1, 0, 131072, 64, 16384, 0,
                                            ctypes.byref(dev), ctypes.byref(host)) == 0
    pool = 16384 * 2 * 16 * 128 * 2            # slots x (K + V) x g_s x d x bf16
    assert dev.value >= 2 * pool and host.value >= 2 * pool
    no_cache = dev.value
    # a warm tier adds its cache to the device buffer only
    assert lib.hga_host_tiered_buffer_bytes(c, 1, 1, 0, 131072, 64, 16384, 20000,
                                            ctypes.byref(dev), ctypes.byref(host)) == 0
    assert dev.value >= no_cache + 20000 * 2 * 16 * 128 * 2
    # a window must hold one query chunk of every (sequence, KV head); so must the cache
    assert lib.hga_host_tiered_buffer_bytes(c, 1, 1, 0, 131072, 64, 4 * gmax - 1, 0,
                                            ctypes.byref(dev), ctypes.byref(host)) == 1
    assert lib.hga_host_tiered_buffer_bytes(c, 1, 1, 0, 131072, 64, 16384, 4 * gmax - 1,
                                            ctypes.byref(dev), ctypes.byref(host)) == 1
    assert lib.hga_host_tiered_buffer_bytes(c, 1, 1, 0, 131072, 64, 16384, -1,
                                            ctypes.byref(dev), ctypes.byref(host)) == 1
    assert lib.hga_host_tiered_buffer_bytes(c, 1, 1, 0, 131072, 0, 16384, 0,
                                            ctypes.byref(dev), ctypes.byref(host)) == 1
    assert lib.hga_host_tiered_buffer_bytes(c, 1, 1, 0, 131072, 64, 16384, 0, None, None) == 1
    # argument errors are reported before any pointer is touched
    stats = H.hga_tier_stats()
    assert lib.hga_attend_host_tiered(c, 1, 1, 16, 0, 131072, None, 131072, 16, 16, 16, None, 256, 0,
                                      256, 0, 64, 16384, 0, 4, None, None, ctypes.byref(stats)) == 1
    assert lib.hga_attend_host_tiered(c, 1, 1, 16, 0, 131072, 16, 131072, 16, 16, 16, None, 256, 0,
                                      256, 0, 64, 16384, 0, -1, None, None, ctypes.byref(stats)) == 1


def test_one_hip_runtime_whatever_the_import_order():
    """Loading the library before torch must not leave two HIP runtimes in the
    process (the library's would then find no device): the binding imports
    torch first, so the library binds to the runtime torch carries."""
    import subprocess
    import sys
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import hierarchical_kv_routing_amd as H\n"
        "H.lib()\n"
        "import torch\n"
        "print(len({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))\n"
    ) % (ROOT,)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout


def test_attend_noalloc_rejects_calls_beyond_its_scratch(lib):
    """hga_attend_noalloc: a call whose split partials exceed the static
    scratch (16 MiB) returns HGA_ERR_WORKSPACE_TOO_SMALL before any HIP call;
    the usual argument checks come first."""
    assert H.attend_noalloc_max_scratch_bytes() == 16 << 20
    # 256 sequences x 4 KV heads of decode with 256 routed whole chunks:
    # 1068 granules, 134 key splits per unit
    cfg = H.Config.from_workload(W.DECODE_64K, n_q_heads=16, top_chunks=256, top_groups=0)
    assert H.attend_workspace_bytes(cfg, 256, 20000, 1) > 16 << 20
    c = ctypes.byref(cfg.c())
    assert lib.hga_attend_noalloc(c, 1, 256, 16, 20000, 1, 16, 16, 20032, 16, 16, 16, None, None) == 3
    assert lib.hga_attend_noalloc(c, 1, 256, None, 20000, 1, 16, 16, 20032, 16, 16, 16, None, None) == 1
    assert lib.hga_attend_noalloc(c, 1, 256, 16, 20000, 0, 16, 16, 20032, 16, 16, 16, None, None) == 0
