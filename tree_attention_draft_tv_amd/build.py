"""Compile the HIP sources into the in-tree shared library ``libtv.so``.

The library is the C ABI declared in ``include/tv.h``; it is built for
gfx950 (MI355X) only. Run ``python -m tree_attention_draft_tv_amd.build``
or call :func:`build`.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libtv.so")

SOURCES = ("tv_api.hip", "tv_mask.hip", "tv_attention.hip", "tv_accept.hip", "tv_commit.hip",
           "tv_linear.hip", "tv_budget.hip")
ARCH = "gfx950"

# Packed-fp32 VALU forms are kept out of the device code on purpose.
COMMON_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE,
    "-I" + CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libtv.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(
        line for line in (res.stdout + res.stderr).splitlines()
        if "packed-fp32-ops' is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (res.returncode, " ".join(cmd), out))
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link ``libtv.so``; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for fut in [ex.submit(_run, c, verbose) for c in cmds]:
            fut.result()
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
