"""Build the in-tree HIP library ulysses_all_re_amd/libua2a.so for gfx950.

    python -m ulysses_all_re_amd.build

The library is compiled with hipcc for MI355X (gfx950) only, from the
sources under csrc/ and the public header include/ua2a.h.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libua2a.so")
SOURCES = [os.path.join(CSRC, "ua2a_kernels.hip"), os.path.join(CSRC, "ua2a_host.cpp")]
HEADERS = [os.path.join(INCLUDE, "ua2a.h"), os.path.join(CSRC, "ua2a_geometry.h"),
           os.path.join(CSRC, "ua2a_bodies.h"), os.path.join(CSRC, "ua2a_internal.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Werror",
    "-Wno-unused-command-line-argument",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def build(verbose: bool = False) -> str:
    """Compile libua2a.so (always recompiles) and return its path."""
    tmp = LIBRARY + ".tmp"
    cmd = [HIPCC, *FLAGS, "-x", "hip", *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
