"""Shared test set-up: the ``gpu`` marker and the repository root on sys.path."""

import pathlib
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))
TESTS = pathlib.Path(__file__).resolve().parent
if str(TESTS) not in sys.path:
    sys.path.insert(0, str(TESTS))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test, skipped unless KDACONV_SLOW=1")


@pytest.fixture(scope="session")
def olib():
    import oracle

    oracle.build()
    return oracle.load()
