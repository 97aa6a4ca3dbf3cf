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

    path = os.environ.get("MUON_PARITY_SUMMARY")
    if path:
        write_parity_summary(path, RECORDS)


def write_parity_summary(path, records):
    """Worst figures per test (markdown table): the asserted metric of each
    mode (bf16 NS: max |dO|; fp32 NS: relative Frobenius error) and the norm
    ratio, over every matrix the test compared."""
    groups = {}
    for r in records:
        groups.setdefault((r.get("test", ""), r.get("ns", "?"), r.get("variant", "?")), []).append(r)
    lines = ["| test | NS | variant | matrices | worst max abs dO | worst rel F dO | worst abs(norm ratio - 1) |",
             "|---|---|---|---:|---:|---:|---:|"]
    for (test, ns, variant), rs in groups.items():
        lines.append(f"| `{test.split('::', 1)[-1]}` ({test.split('::', 1)[0].split('/')[-1]}) | {ns} | {variant} | "
                     f"{len(rs)} | {max(r['max_abs_dO'] for r in rs):.2e} | {max(r['rel_F_dO'] for r in rs):.2e} | "
                     f"{max(abs(r['norm_ratio_m1']) for r in rs):.2e} |")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
