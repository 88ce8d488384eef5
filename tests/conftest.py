"""pytest configuration: the ``gpu`` marker and shared fixtures.

Tests marked ``gpu`` need an MI355X (gfx950) and the built HIP library; every
other test runs on the CPU only.
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


def golden_rows(name):
    """Non-comment, non-empty lines of a golden fixture, split on whitespace."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


@pytest.fixture
def tune():
    """Pins library choices through skgemm_set_override for one test
    (``tune("kind", 1)``); every knob is restored to the library's own
    choice afterwards."""
    import split_reduction_amd as sk

    def set_(name, value):
        sk.skgemm_set_override(name, int(value))

    try:
        yield set_
    finally:
        sk.clear_overrides()
