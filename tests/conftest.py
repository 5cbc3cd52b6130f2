"""Shared pytest set-up: the ``gpu`` marker and repository paths.

Tests marked ``gpu`` need a real MI355X and call the library through its C ABI;
everything else runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    if not os.path.exists(oracle.oracle_lib_path()):
        oracle.build_oracle()
    return oracle.load_library()
