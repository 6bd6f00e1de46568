"""Shared pytest configuration: the `gpu` marker and the repository root on
sys.path (so `oracle`, `workloads` and the package import without install)."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Score parity report: the condition-scaled error (asserted <= 1e-5) and
    the plain relative error over scores of at least 1e-2 of the rms, worst
    case over every score check of the run."""
    mod = sys.modules.get("tests._parity")
    rows = getattr(mod, "PLAIN_REPORT", []) if mod is not None else []
    if not rows:
        return
    n = sum(r[1] for r in rows)
    wc = max(rows, key=lambda r: r[2])
    wp = max(rows, key=lambda r: r[3])
    terminalreporter.write_line(
        f"score parity over {len(rows)} checks: worst |err| / (||k|| sum|LUT|) = {wc[2]:.3e} "
        f"({wc[0]}); plain |err| / |s| over {n} scores with |s| >= 1e-2 rms: worst {wp[3]:.3e} "
        f"({wp[0]})")
