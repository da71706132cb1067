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
def _oracle_built():
    import oracle
    oracle.build(force=not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")))
    yield
