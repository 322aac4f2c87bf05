"""Shared test set-up.

Markers: ``gpu`` (needs an MI355X; run with ``-m gpu``) and ``slow``.
Tests that are not marked ``gpu`` run on a CPU-only machine.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


@pytest.fixture(scope="session")
def ref():
    """The CPU oracle (built on first use)."""
    import oracle
    return oracle.default()
