"""Shared pytest configuration: the ``gpu`` marker and common fixtures."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")
    config.addinivalue_line("markers", "slow: long CPU oracle runs")


def pytest_collection_modifyitems(config, items):
    # A gpu-marked test on a machine without a GPU is a configuration error, not a skip: fail loudly
    # only when gpu tests were explicitly selected; otherwise leave selection to -m.
    pass
