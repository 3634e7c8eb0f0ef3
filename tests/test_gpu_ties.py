"""Exact score ties on the GPU: the lowest index wins (top-K selection of the
xllm-io page, section 3, with the tie rule fixed for this path).

Raw keys of every chunk past the sinks are zero except a few "live" chunks,
so the summaries of the zero chunks are exactly 0 and every query scores
them exactly 0: they tie with each other at the K-th place (in the mixed
cases the live chunks score above them).  The oracle's margin there is
exactly 0, which parity.compare_routes does not accept as a near-tie: the
GPU's chunk and group lists must equal the oracle's lowest-index choice.
Covered: the fused prefill routing (rank select, <= 512 candidates), with
and without the screened chunk scoring, the block radix select (> 512
middle chunks) and the segmented decode scoring,
where each segment keeps its own winners and the merge must still prefer
the lower index across segments.
"""
import numpy as np
import pytest

import hierarchical_kv_routing_amd as H
import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu

CASES = {
    # fused prefill routing: 64 query chunks x 4 KV heads, rank select
    "prefill_mixed": (W.QWEN3_PREFILL.scaled(n_ctx=4096, kv_cap=4096, n_q=4096, planted=0), (5, 9, 17, 22)),
    "prefill_all_zero": (W.QWEN3_PREFILL.scaled(n_ctx=4096, kv_cap=4096, n_q=4096, planted=0), ()),
    # the same shape over 12288 tokens: units past query chunk 74 have more
    # than 64 middle chunks, so their chunk scoring is screened (hi*hi, then
    # the split products of the chunks left in contention: every tied zero
    # chunk stays in contention)
    "prefill_screened_mixed": (W.QWEN3_PREFILL.scaled(n_ctx=12288, kv_cap=12288, n_q=12288, planted=0),
                               (5, 40, 90, 150)),
    "prefill_screened_all_zero": (W.QWEN3_PREFILL.scaled(n_ctx=12288, kv_cap=12288, n_q=12288, planted=0),
                                  ()),
    # one query chunk after 624 closed chunks: 614 middle chunks, radix select
    "radix_mixed": (W.QWEN3_PREFILL.scaled(n_ctx=40000, kv_cap=40000, q_pos0=39936, n_q=64, planted=0),
                    (100, 300, 500)),
    # decode shape: 2 sequences x 4 KV heads, 502 middle chunks in 8 segments
    "decode_segmented_mixed": (W.DECODE_64K.scaled(batch=2, n_ctx=32769, kv_cap=32832, q_pos0=32768,
                                                   planted_per_q_head=0), (20, 100, 300)),
    "decode_segmented_all_zero": (W.DECODE_64K.scaled(batch=2, n_ctx=32769, kv_cap=32832, q_pos0=32768,
                                                      planted_per_q_head=0), ()),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_exact_ties_lowest_index_wins(name):
    w, live = CASES[name]
    print(f"[gpu] ties {name}: {w}", flush=True)
    q, k, v = P.make_inputs_parallel(w, seed=3)
    C = w.chunk_size
    keep = np.zeros(w.kv_cap // C, bool)
    keep[: w.n_sink_chunks] = True
    keep[list(live)] = True
    k = k.reshape(w.batch, w.n_kv_heads, -1, C, w.head_dim)
    k[:, :, ~keep] = 0.0
    k = k.reshape(w.batch, w.n_kv_heads, w.kv_cap, w.head_dim)
    cfg = H.Config.from_workload(w)
    if name.startswith("decode"):
        assert H.route_workspace_bytes(cfg, w.batch, w.q_pos0, w.n_q) > 0  # segmented scoring
    run = P.DeviceRun(w, q, k, v)
    units = P.all_units(w)
    orc = P.oracle_route(run, q, k, units)
    exact, near = P.compare_routes(run, orc, units, name=f"ties:{name}")
    assert near == 0 and exact == len(units)
    info = [orc["info"][u] for u in units]
    tied_c = sum(1 for x in info if x["margin_c"] == 0)
    tied_g = sum(1 for x in info if x["margin_g"] == 0)
    print(f"[gpu] ties {name}: {len(units)} units, chunk-level ties {tied_c}, group-level {tied_g}",
          flush=True)
    # fewer live chunks than K_c: wherever more than K_c + |live| chunks
    # compete, the K-th and the next candidate are both zero chunks (a tie)
    crowded = sum(1 for x in info if len(x["mid"]) > w.top_chunks + len(live))
    assert crowded >= 1 and tied_c >= crowded and tied_g >= 1
    if not live:
        # all middle chunks tie: the K_c lowest middle chunks, then the K_g
        # lowest of their groups
        ci = run.np("chunk_idx")
        t0 = w.q_pos0 // C
        for (b, h, t) in units:
            mids = info[units.index((b, h, t))]["mid"]
            want = mids[: min(w.top_chunks, len(mids))]
            got = [int(x) for x in ci[b, h, t - t0] if x >= 0]
            assert got == want, ((b, h, t), got, want)
    P.check_attention(run, q, k, v, P.sample_units(w, 8), name=f"ties:{name}")
