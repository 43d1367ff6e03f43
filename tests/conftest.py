"""Shared pytest setup: markers, import path, build-on-demand of the oracle."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Stress mode (more seeds, exhaustive codec sweeps), as TK_FULL_TEST=1.
FULL = os.environ.get("TK_FULL_TEST", "0") not in ("", "0")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size) case")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle
