import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Error statistics of the full-size parity checks (max / mean absolute error per
    compared tensor against the fp64 oracle)."""
    try:
        from _parity import STATS
    except ImportError:
        return
    rows = [s for s in STATS if s.get("report")]
    if not rows:
        return
    tr = terminalreporter
    tr.section("parity against the fp64 oracle (full-size workloads)")
    for s in rows:
        extra = ""
        if "max_err_over_bound" in s:
            extra = f" err/bound {s['max_err_over_bound']:.3f}"
        if "rel" in s:
            extra = f" rel {s['rel']:.2e}"
        tr.write_line(f"{s['what']:<28} n={s['n']:>11} max_abs={s['max_abs']:.3e} "
                      f"mean_abs={s['mean_abs']:.3e} max|ref|={s['max_ref']:.3g}{extra}")
