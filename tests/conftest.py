import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes tens of seconds on the CPU")


def pytest_terminal_summary(terminalreporter):
    """Achieved parity margins of the run: per test, the worst max-abs and rel-L2 of its
    comparisons with the oracle, each also as a fraction of its bar."""
    h = sys.modules.get("harness")
    if h is None or not getattr(h, "MARGINS", None):
        return
    worst = {}
    for test, what, err, rel, bar_abs, bar_rel in h.MARGINS:
        w = worst.setdefault(test, [0, 0.0, 0.0, bar_abs, bar_rel, ""])
        w[0] += 1
        if rel / bar_rel >= w[2] / w[4]:
            w[5] = what
        w[1] = max(w[1], err)
        w[2] = max(w[2], rel)
    tr = terminalreporter
    tr.write_sep("-", "parity margins (worst comparison per test: max-abs, rel-L2, fraction of the bar)")
    for test, (n, err, rel, bar_abs, bar_rel, what) in sorted(worst.items()):
        tr.write_line(f"{test}: {n} cmp, max-abs {err:.2e} ({err / bar_abs:.0%}), rel-L2 {rel:.2e} "
                      f"({rel / bar_rel:.0%}), worst: {what}")
