"""Build the host emulation of the ua2a library (tests only).

libua2a_emu.so = the library's own host logic (ua2a_host.cpp) + a backend
that runs the kernels' per-thread bodies on the CPU (emu_backend.cpp),
compiled with g++ (no device code).  With sanitize=True the build adds
AddressSanitizer and UndefinedBehaviorSanitizer (host code only).
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "ulysses_all_re_amd", "csrc")
SOURCES = [os.path.join(HERE, "emu_backend.cpp"), os.path.join(CSRC, "ua2a_host.cpp")]


def library_path(sanitize: bool = False) -> str:
    return os.path.join(HERE, "libua2a_emu_asan.so" if sanitize else "libua2a_emu.so")


def build(sanitize: bool = False) -> str:
    out = library_path(sanitize)
    cmd = ["g++", "-std=c++17", "-O1" if sanitize else "-O2", "-g", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-Werror", "-Wno-unused-parameter", "-Wno-unknown-pragmas",
           # the bodies keep per-lane vectors in arrays written and read under the
           # same per-lane guard (ok[k]), which gcc's flow analysis cannot pair up
           "-Wno-maybe-uninitialized",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    if sanitize:
        cmd += ["-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                "-fno-sanitize-recover=undefined"]
    cmd += [*SOURCES, "-o", out + ".tmp"]
    subprocess.check_call(cmd)
    os.replace(out + ".tmp", out)
    return out


def asan_runtime() -> str:
    return subprocess.check_output(["g++", "-print-file-name=libasan.so"], text=True).strip()


if __name__ == "__main__":
    print(build())
    print(build(sanitize=True))
