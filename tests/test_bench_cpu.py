"""bench.py's host-side logic, on the CPU: the one-GPU refusal and the parsing of
kernel names in rocprofv3 output."""
from __future__ import annotations

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert "ONE GPU" in res.stderr and res.stdout == ""


def test_mode_of_a_kernel_name():
    assert not bench._is_mode1("void ua2a::ua2a_direct3d_kernel<16, false, false>(ua2a::DirectGeom)")
    assert bench._is_mode1("void ua2a::ua2a_direct3d_kernel<16, true, false>(ua2a::DirectGeom)")
    assert bench._is_mode1("void ua2a::ua2a_direct_kernel<8, true, true>(ua2a::DirectGeom)")
    assert not bench._is_mode1("_ZN4ua2a20ua2a_direct3d_kernelILi16ELb0ELb1EEEvNS_10DirectGeomE")
    assert bench._is_mode1("_ZN4ua2a20ua2a_direct3d_kernelILi16ELb1ELb0EEEvNS_10DirectGeomE")
    assert not bench._is_mode1("__amd_rocclr_copyBuffer")
