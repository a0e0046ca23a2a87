"""Shared test setup.

Markers: ``gpu`` -- the test needs an MI355X (HIP device) and calls the HIP
library through its C ABI; everything else runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU; calls libzeroshard's HIP kernels")


def _ensure_host_built():
    """Load what is built; build a host library only when it is missing."""
    from sharded_mixed_precision_zs_amd import build as pkg_build
    import oracle.build as oracle_build
    if not os.path.exists(oracle_build.LIB):
        oracle_build.build()
    if not os.path.exists(pkg_build.SYNTH_HOST):
        pkg_build.build_synth_host()


_ensure_host_built()


@pytest.fixture(scope="session")
def hip_built():
    """The HIP libraries (built here, from source, only if missing)."""
    from sharded_mixed_precision_zs_amd import build as pkg_build
    if not all(os.path.exists(p) for p in (pkg_build.LIB, pkg_build.SYNTH_DEV, pkg_build.COPY,
                                           pkg_build.VARIANTS)):
        pkg_build.build_all()
    return pkg_build


def golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def golden():
    return golden_rows
