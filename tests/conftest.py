"""Shared test set-up: the `gpu` marker, and in-place builds of the CPU-side
libraries (oracle, input generators) when they are missing."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _cpu_libs():
    import oracle
    from activation_residual_compression_amd import synth
    oracle.build(force=False)
    synth.build(force=False)
