import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Report every route and attention comparison of the run (near-tie
    counts, max-abs against exact and against bf16-cached keys, rows above
    the max-abs bar); also written to gpurun_out/parity_records.json when
    that folder exists."""
    mod = sys.modules.get("tests.parity")
    recs = getattr(mod, "RECORDS", None) if mod else None
    if not recs:
        return
    tr = terminalreporter
    tr.section("parity records")
    for r in recs:
        if r["kind"] == "routes":
            tr.write_line(f"routes    {r['name']}: units={r['units']} exact={r['exact']} "
                          f"near_tie={r['near_tie']} exact_ties={r['exact_ties']}")
        else:
            extra = ""
            if "max_abs_cached_keys" in r:
                extra = (f" | cached keys max_abs={r['max_abs_cached_keys']:.3g}"
                         f" rel_l2={r['rel_l2_cached_keys']:.3g} | bound ratio {r['bound_ratio_max']:.3g}")
            tr.write_line(f"attention {r['name']}: rows={r['rows']} exact keys max_abs={r['max_abs']:.3g} "
                          f"rel_l2={r['rel_l2']:.3g} rows>tol={r['rows_over_abs_tol']}{extra}")
    out = os.path.join(ROOT, "gpurun_out")
    if os.path.isdir(out):
        with open(os.path.join(out, "parity_records.json"), "w") as f:
            json.dump(recs, f, indent=1)
