"""Build the C-ABI test programs (tests/c_abi/ua2a_consumer, tests/c_abi/ua2a_graph)
with gcc against include/ua2a.h and libua2a.so."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "ulysses_all_re_amd")
BINARY = os.path.join(HERE, "ua2a_consumer")
GRAPH_BINARY = os.path.join(HERE, "ua2a_graph")


def build(name: str = "ua2a_consumer") -> str:
    binary = os.path.join(HERE, name)
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", "-I/opt/rocm/include",
           os.path.join(HERE, name + ".c"), "-o", binary + ".tmp",
           f"-L{PKG}", "-lua2a", f"-Wl,-rpath,{PKG}", "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib"]
    subprocess.check_call(cmd)
    os.replace(binary + ".tmp", binary)
    return binary


if __name__ == "__main__":
    print(build())
    print(build("ua2a_graph"))
