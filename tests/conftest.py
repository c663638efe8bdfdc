import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # Build the HIP library only when nothing is built yet.
    lib = os.path.join(ROOT, "tree_attention_draft_tv_amd", "libtv.so")
    if not os.path.exists(lib):
        from tree_attention_draft_tv_amd import build as _build
        _build.build()


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
