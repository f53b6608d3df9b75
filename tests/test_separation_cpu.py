"""The product path and the CPU oracle stay apart.

The package (the HIP library, its host code and the Python binding) must not
name, import, link or load the oracle: only the tests, the smoke check and the
benchmark's CPU-baseline leg may.  These checks run on the CPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "ulysses_all_re_amd")


def test_package_sources_never_name_the_oracle():
    hits = []
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".cpp", ".h", ".hip", ".c")):
                path = os.path.join(dirpath, f)
                with open(path, encoding="utf-8") as fh:
                    for n, line in enumerate(fh, 1):
                        if "oracle" in line.lower():
                            hits.append(f"{os.path.relpath(path, ROOT)}:{n}")
    assert not hits, hits


def test_loading_the_library_loads_no_oracle():
    """A fresh interpreter imports the package and loads libua2a.so; neither
    the oracle module nor its shared library is then present."""
    code = (
        "import sys, ulysses_all_re_amd as ua\n"
        "ua.load_library()\n"
        "ua.ua2a_layout(8, 1, 9450, 40, 128, 2)\n"
        "maps = open('/proc/self/maps').read()\n"
        "assert 'libua2a.so' in maps, 'library not mapped'\n"
        "assert 'oracle' not in maps, 'oracle library mapped'\n"
        "assert not any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules), 'oracle imported'\n"
        "print('ok')\n"
    )
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout + res.stderr


def test_library_does_not_link_the_oracle():
    import ulysses_all_re_amd as ua
    res = subprocess.run(["readelf", "-d", ua.LIBRARY], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stderr
    needed = [l for l in res.stdout.splitlines() if "NEEDED" in l]
    assert needed and not any("oracle" in l for l in needed), needed
