import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Per-case parity counts of the GPU tests (outside pytest's output
    capture, so that they stay in the log of a quiet run)."""
    mod = sys.modules.get("tests.parity")
    recs = getattr(mod, "RECORDS", None) if mod else None
    if not recs:
        return
    tr = terminalreporter
    tr.section("parity counts (units = (row, group) pairs; every unit's attention compared)")
    tr.write_line(f"{'case':42s} {'units':>7s} {'identical':>9s} {'tie band':>8s} "
                  f"{'score err/bound':>15s} {'attn max-abs':>12s}")
    for r in recs:
        tr.write_line(f"{r['case'][:42]:42s} {r['units']:7d} {r['identical']:9d} "
                      f"{r['tie_band']:8d} {r['score_err_of_bound']:15.3f} "
                      f"{r['attn_max_abs']:12.2e}")
