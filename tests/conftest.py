"""Shared pytest configuration.

Markers: `gpu` -- needs an MI355X (gfx950) and the built HIP library; the
CPU suite runs with `-m "not gpu"`.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _libraries_built():
    """Build the oracle (gcc), on a machine with hipcc the HIP library, and
    the C client of the library, if they are missing; an existing build is
    used as it is."""
    import oracle
    oracle.build(force=not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")))
    lib = os.path.join(ROOT, "fsdp_sharded_state_amd", "libfsstate.so")
    if not os.path.exists(lib) and os.path.exists("/opt/rocm/bin/hipcc"):
        from fsdp_sharded_state_amd import build as _b
        _b.build()
    if os.path.exists(lib):
        sys.path.insert(0, os.path.join(ROOT, "tests", "c"))
        import build_client
        build_client.build(force=False)
    yield
