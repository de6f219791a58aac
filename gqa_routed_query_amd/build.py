"""Build libgqa.so (HIP, gfx950) in place, next to this file.

Usage: ``python gqa_routed_query_amd/build.py`` (run as a script: the package
itself cannot be imported before the library exists), or ``build()`` from
``__graft_entry__``. Only the standard library is imported here.
The library is compiled with hipcc for gfx950 only. Packed fp32 instructions
are disabled for all device code (``-packed-fp32-ops``); the host pass warns
that it does not know that target feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libgqa.so")
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libgqa)")
    return path


def build_command(out: str = LIB_PATH) -> list[str]:
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-result",
        "-I", INCLUDE, "-I", CSRC,
        *sources, "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libgqa.so; returns the library path."""
    tmp = LIB_PATH + ".tmp"
    cmd = build_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
