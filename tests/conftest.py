"""Shared pytest set-up: the ``gpu`` marker, import paths, and built libraries.

Tests marked ``gpu`` need a real MI355X; everything else runs on the CPU. The fp64 oracle and
the GPU library are built if (and only if) no build is present yet.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.load()
