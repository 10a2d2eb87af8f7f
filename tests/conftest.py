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
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Combined excusal accounting of every GPU parity test that ran."""
    try:
        from gpu_util import SESSION
    except Exception:
        return
    if SESSION["total"] == 0:
        return
    t, e, n = SESSION["total"], SESSION["excused"], SESSION["near"]
    terminalreporter.write_line(
        f"[parity] {t} request-cycles compared with the oracle: {e} excused mismatches "
        f"(rate {e / t:.2e}, bar 1e-4), {n} near-threshold request-cycles (margin < 1e-6, rate {n / t:.2e})")
