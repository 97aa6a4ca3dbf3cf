import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Per-matrix parity figures of every GPU-vs-oracle comparison of the
    session (so that a quiet run still shows them)."""
    try:
        from parity import RECORDS
    except Exception:
        return
    if not RECORDS:
        return
    tr = terminalreporter
    tr.write_sep("-", f"parity figures ({len(RECORDS)} matrices)")
    for r in RECORDS:
        extra = f" div {r['div_dO']:.2e}" if "div_dO" in r else ""
        tr.write_line(f"{r['case']}: max|dO| {r['max_abs_dO']:.3e} relF {r['rel_F_dO']:.2e} "
                      f"||O||ratio-1 {r['norm_ratio_m1']:+.2e} max|O| {r['max_abs_O']:.3f}{extra}")
