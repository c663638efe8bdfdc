import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # Build the HIP library when it is missing or older than any of its
    # sources or the public header (a stale library would test old code).
    from tree_attention_draft_tv_amd import build as _build
    lib = _build.LIB_PATH
    srcs = [os.path.join(_build.CSRC, f) for f in os.listdir(_build.CSRC)]
    srcs.append(os.path.join(_build.INCLUDE, "tv.h"))
    if not os.path.exists(lib) or \
            os.path.getmtime(lib) < max(os.path.getmtime(f) for f in srcs):
        _build.build()


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
