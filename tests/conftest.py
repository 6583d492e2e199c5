"""Shared pytest configuration.

Tests marked ``gpu`` run the HIP library through its C ABI on a gfx950 device and
compare against the CPU oracle; every other test runs on the CPU only.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def pytest_sessionfinish(session, exitstatus):
    """Report the largest parity errors the GPU tests measured (output per-row
    relative error and lse absolute error, per path)."""
    mod = sys.modules.get("gpu_helpers")
    if mod is not None and any(v[0] or v[1] for v in mod.MAX_ERR.values()):
        for path, (o, l) in mod.MAX_ERR.items():
            print(f"\nlargest parity errors ({path}): output {o:.3e}, lse {l:.3e}", flush=True)
