import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Every attention comparison of the session (max ulp, share within 2
    bf16 ulp, worst absolute and relative error), so the figures show even
    under -q."""
    try:
        import parity
    except ImportError:
        return
    if not parity.REPORTS:
        return
    tr = terminalreporter
    tr.section("attention parity (GPU against the oracle)")
    worst = min(r["frac_within_2ulp"] for _, r in parity.REPORTS)
    tr.write_line(f"{len(parity.REPORTS)} comparisons; lowest share within 2 bf16 ulp "
                  f"{worst:.5f} (floor {parity.MIN_WITHIN_2ULP})")
    for what, r in parity.REPORTS:
        tr.write_line(f"  {what}: n={r['n']} max_ulp={r['max_ulp']:.1f} "
                      f"within_2ulp={r['frac_within_2ulp']:.5f} max_abs={r['max_abs']:.2e} "
                      f"max_rel(|o|>1e-6)={r['max_rel_nonzero']:.2e} fail={r['fail']}")
