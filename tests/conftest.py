import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size configuration (minutes of host work)")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """How many fp16/bf16 weights the parity tests checked, and how many lay beyond 1 ulp."""
    gu = sys.modules.get("gpu_util")
    if gu is not None and gu.ULP_STATS["weights"]:
        st = gu.ULP_STATS
        terminalreporter.write_line(
            f"fp16/bf16 weights checked: {st['weights']}, beyond 1 ulp: {st['beyond_1ulp']}, "
            f"largest distance: {st['max_ulp']} ulp")
