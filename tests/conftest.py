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
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large full-size cases")


def pytest_collection_modifyitems(config, items):
    """GPU tests run only against a libekv.so built from the sources in this tree."""
    if any(item.get_closest_marker("gpu") for item in items):
        try:
            from mixed_precision_paged_amd import build
            build.check_library_matches_sources()
        except ImportError:  # libekv.so absent: the GPU tests fail loudly on import
            return
