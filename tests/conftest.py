"""Shared pytest configuration.

Tests marked ``gpu`` need an MI355X (gfx950) and the built native library;
everything else runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_rows(name):
    """Data rows of a golden fixture: comment lines (#) and blanks dropped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


_WORKLOADS = {}


@pytest.fixture(scope="session")
def decode_workload():
    """Cached seeded decode workloads (generation of the big ones takes a while)."""
    from mla_attention_nvfp4_amd import workloads

    def get(n, H=None):
        key = (n, H)
        if key not in _WORKLOADS:
            print(f"  generating decode workload {n} (H={H})", flush=True)
            _WORKLOADS[key] = workloads.decode_workload(n, H)
        return _WORKLOADS[key]

    return get
