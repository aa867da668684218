"""Shared pytest configuration.

Tests marked ``gpu`` need an MI355X (gfx950) and the built HIP library; every
other test runs on the CPU alone.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: large oracle runs (minutes of CPU time)")


@pytest.fixture(scope="session")
def oracle_threads():
    """Worker threads for oracle runs: at most 16, never more than the CPUs
    this process may use."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))
