"""bench.py's host-side logic, on the CPU: the one-GPU refusal, the parsing of
kernel names in rocprofv3 output and the records' threaded oracle timing."""
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


def test_threaded_oracle_equals_the_single_thread_oracle():
    """The records' multi-thread oracle timing splits the senders over threads;
    its output must be the single-thread oracle's, byte for byte."""
    import numpy as np

    import oracle
    rng = np.random.default_rng(3)
    for (w, B, S, H, D, dt) in [(1, 2, 3, 4, 5, np.uint16), (3, 2, 5, 6, 4, np.uint32),
                                (8, 1, 7, 16, 3, np.uint8), (5, 2, 4, 10, 2, np.uint64)]:
        for mode in (0, 1):
            shape = (w, B, S, H, D) if mode == 0 else (w, B, S * w, H // w, D)
            x = rng.integers(0, np.iinfo(dt).max, size=shape, dtype=dt)
            got, secs, threads = bench.oracle_on_threads(x, mode, w)
            assert threads == min(w, bench.HOST_CPU_SHARE, os.cpu_count() or 1) and secs >= 0
            assert np.array_equal(got, oracle.exchange(x, mode, w)), (w, mode)


def test_cpu_baseline_reports_one_thread_and_all_cores():
    import torch

    from workloads import make_tensor
    x = make_tensor((4, 1, 64, 8, 16), "bf16", "normal", 0)
    moved = 2 * x.numel() * 2
    cb = bench.cpu_baseline(x, 4, 2, moved, "small")
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["value"] > 0
    assert cb["nproc"] == os.cpu_count() and cb["cpu_model"]
    allc = cb["all_cores"]
    assert allc["kind"] == "oracle" and allc["value"] > 0
    assert allc["cores"] == min(4, bench.HOST_CPU_SHARE, os.cpu_count() or 1)
    assert isinstance(x, torch.Tensor)
