"""Shared test configuration.

Tests marked ``gpu`` need an MI355X and call the HIP library through its
C ABI; everything else runs on the CPU.
"""

import json
import os

import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def golden():
    return load_golden
