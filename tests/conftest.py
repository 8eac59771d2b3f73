"""Shared pytest configuration.

Markers: ``gpu`` tests need an MI355X and the built HIP library; everything
else runs on the CPU. Fixture files under tests/golden are YAML, each carrying
the citation for its values.
"""
import os
import sys

import pytest
import yaml

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: longer CPU test")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return yaml.safe_load(f)


@pytest.fixture
def golden():
    return load_golden
