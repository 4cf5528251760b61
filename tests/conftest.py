import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running check")


def pytest_terminal_summary(terminalreporter):
    """Wall time of each full-size oracle run (every (sequence, kv head) pair
    of a workload), so that the cost of complete parity stays visible."""
    mod = sys.modules.get("tests.gpu_util")
    times = getattr(mod, "ORACLE_TIMES", None) if mod else None
    if not times:
        return
    terminalreporter.write_sep("-", "oracle wall time per full-size check")
    for label, pairs, sec, threads in times:
        terminalreporter.write_line(f"{label}: {pairs} pairs, {sec:.1f} s on {threads} threads")
