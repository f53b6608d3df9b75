"""The no-allocation entry point, ua2a_exchange_chunked_noalloc: a chunked
exchange through the library's own static device window, for callers that
cannot allocate.  Its output must equal ua2a_exchange's chunked output
through a caller-owned window, byte for byte, and the oracle's.

CPU tests run the library's host logic with the kernel bodies in the host
emulation; GPU tests call the real library through the C ABI, two calls in a
row with the second on a smaller input (the shared window keeps the first
call's bytes, which the second must not depend on).
"""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import ulysses_all_re_amd as ua
from tests.test_emulated_kernels import Buf, _load, oracle_bytes, rand_bytes, ua2a_layout
from workloads import BITS_VIEW, make_tensor

DEV = "cuda:0"


# ------------------------------------------------------------ host emulation

@pytest.fixture(scope="module")
def emu():
    return _load()


def _emu_pair(lib, shape, mode, path=ua.UA2A_PATH_AUTO, seed=0):
    """(input bytes, output of the no-allocation call, output through a
    caller-owned window, launch info) for one shape on the emulated library."""
    w, B, S, H, D, e = shape
    lay = ua2a_layout(lib, w, B, S, H, D, e)
    n = lay.tensor_bytes
    xin, y_noalloc, y_window = Buf(n), Buf(n), Buf(n)
    win = Buf(lay.window_bytes)
    xin.view[:] = rand_bytes(n, seed)
    h = ctypes.c_void_p()
    assert lib.ua2a_plan(ctypes.byref(h), w, B, S, H, D, e, 0, win.ptr, lay.window_bytes, 0) == 0
    try:
        assert lib.ua2a_plan_set_path(h, path) == 0
        info = ua.ua2a_launch_info_t()
        assert lib.ua2a_describe(h, mode, 1, xin.ptr, y_window.ptr, ctypes.byref(info)) == 0
        lib.ua2a_emu_reset_counts()
        rc = lib.ua2a_exchange_chunked_noalloc(h, mode, xin.ptr, y_noalloc.ptr, None)
        assert rc == 0, (rc, lib.ua2a_plan_last_error(h))
        assert lib.ua2a_emu_launches() == info.launches
        assert lib.ua2a_exchange(h, mode, 1, xin.ptr, y_window.ptr, None) == 0
    finally:
        lib.ua2a_destroy(h)
    assert all(b.guards_intact() for b in (xin, y_noalloc, y_window, win))
    return xin.view.copy(), y_noalloc.view.copy(), y_window.view.copy(), info


@pytest.mark.parametrize("shape", [(4, 4, 32, 16, 64, 2), (2, 1, 8, 4, 16, 2), (3, 2, 5, 6, 4, 4),
                                   (3, 5, 7, 3, 7, 2), (8, 2, 13, 40, 128, 2)],
                         ids=lambda s: "x".join(map(str, s)))
def test_emulated_noalloc_equals_the_window_exchange(emu, shape):
    """Both one-launch chunked kernels (direct and LDS path), both modes,
    then a second, smaller call."""
    for path in (ua.UA2A_PATH_AUTO, ua.UA2A_PATH_DIRECT, ua.UA2A_PATH_LDS):
        for mode in (0, 1):
            for s in (shape, (2, 2, 3, 4, 8, shape[5])):          # the second call is smaller
                x, got, ref, info = _emu_pair(emu, s, mode, path, seed=mode + 3)
                assert np.array_equal(got, ref), (s, mode, path)
                assert np.array_equal(got, oracle_bytes(x, s, mode)), (s, mode, path)


def test_emulated_noalloc_errors(emu):
    # a one-plane window beyond the library's own: CAPACITY, nothing launched
    w, B, S, H, D, e = 8, 1, 9450, 40, 128, 2
    h = ctypes.c_void_p()
    assert emu.ua2a_plan(ctypes.byref(h), w, B, S, H, D, e, 0, None, 0, 0) == 0
    base = 1 << 40
    emu.ua2a_emu_reset_counts()
    assert emu.ua2a_exchange_chunked_noalloc(h, 0, base, base + (1 << 31), None) == ua.UA2A_ERR_CAPACITY
    assert emu.ua2a_exchange_chunked_noalloc(h, 2, base, base + (1 << 31), None) == ua.UA2A_ERR_INVALID_ARG
    assert emu.ua2a_exchange_chunked_noalloc(h, 0, base, base + 16, None) == ua.UA2A_ERR_ALIAS
    assert emu.ua2a_exchange_chunked_noalloc(None, 0, base, base + (1 << 31), None) == ua.UA2A_ERR_INVALID_ARG
    assert emu.ua2a_emu_launches() == 0
    emu.ua2a_destroy(h)
    # the largest accepted window, and the wrong device
    lay = ua2a_layout(emu, 4, 1, 1024, 16, 1024, 1)
    assert lay.window_bytes == ua.UA2A_NOALLOC_WINDOW_BYTES
    assert emu.ua2a_plan(ctypes.byref(h), 4, 2, 1024, 16, 1024, 1, 0, None, 0, 1) == 0
    assert emu.ua2a_exchange_chunked_noalloc(h, 0, base, base + (1 << 31), None) == ua.UA2A_ERR_DEVICE
    emu.ua2a_destroy(h)


# ----------------------------------------------------------------- the GPU

def note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def bits(t):
    return t.view(BITS_VIEW[t.element_size()])


def _gpu_pair(shape, dtype, mode, mis=0, seed=0):
    w, B, S, H, D = shape
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]
    e = torch.empty((), dtype=dt).element_size()
    lay = ua.ua2a_layout(w, B, S, H, D, e)
    window = torch.empty(lay["window_bytes"], dtype=torch.uint8, device=DEV)
    with_window = ua.Plan(w, B, S, H, D, dt, window=window, device=DEV)
    bare = ua.Plan(w, B, S, H, D, dt, device=DEV)         # no window of its own
    n = w * B * S * H * D
    ishape = (w, B, S, H, D) if mode == 0 else (w, B, S * w, H // w, D)
    x = make_tensor(ishape, dtype, "bytes", seed)
    xin = torch.zeros(n + 8, dtype=dt, device=DEV)
    xin[mis:mis + n] = x.reshape(-1).to(DEV)
    xi = xin[mis:mis + n].view(ishape)
    obuf = torch.full((n + 8,), -1, dtype=BITS_VIEW[e], device=DEV).view(dt)
    got = obuf[mis:mis + n].view(bare.out_shape(mode))
    ref = torch.full(bare.out_shape(mode), -1, dtype=BITS_VIEW[e], device=DEV).view(dt)
    note(f"noalloc {shape} {dtype} mode {mode} mis {mis} {with_window.describe(xi, mode, True, out=got)}")
    bare.exchange_noalloc(xi, mode, got)
    with_window.exchange(xi, mode, True, out=ref)
    torch.cuda.synchronize()
    assert torch.equal(bits(got.cpu()), bits(ref.cpu())), (shape, mode, mis)
    want = oracle.exchange(bits(x).numpy(), mode, w)
    assert np.array_equal(bits(got.cpu()).numpy(), want), (shape, mode, mis)
    guard = bits(obuf.cpu())
    assert (guard[:mis] == -1).all() and (guard[mis + n:] == -1).all()
    bare.close()
    with_window.close()


@pytest.mark.gpu
@pytest.mark.parametrize("first,second", [
    (((4, 4, 2048, 16, 64), "fp16"), ((2, 3, 100, 4, 32), "bf16")),      # the 4-plane workload, then smaller
    (((3, 2, 4681, 12, 80), "fp32"), ((3, 2, 41, 3, 5), "fp32")),         # 54 MB window, then an odd shape
    (((2, 1, 8, 4, 16), "bf16"), ((2, 1, 5, 2, 16), "bf16")),            # short runs: the LDS path (offset output: pieces)
    (((8, 4, 1024, 8, 32), "bf16"), ((3, 4, 8, 3, 7), "bf16")),          # the chunked LDS kernel, 64 B then 14 B runs
], ids=["chunked-then-small", "awkward-then-odd", "tiny-then-tinier", "lds-then-odd"])
def test_noalloc_matches_the_window_exchange(first, second):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    for mode in (0, 1):
        _gpu_pair(*first, mode, seed=40 + mode)
        _gpu_pair(*second, mode, seed=50 + mode)          # the window still holds the first call's bytes
        _gpu_pair(*second, mode, mis=2 if second[1] != "fp32" else 1, seed=60 + mode)   # narrower vectors


@pytest.mark.gpu
def test_noalloc_rejects_a_window_beyond_its_own():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    plan = ua.Plan(8, 1, 9450, 40, 128, torch.bfloat16, device=DEV)     # a 774 MB plane
    base = 1 << 40
    with pytest.raises(ua.UA2AError) as e:
        ua.ua2a_exchange_chunked_noalloc(plan.handle, 0, base, base + (1 << 31), 0)
    assert e.value.code == ua.UA2A_ERR_CAPACITY
    assert plan.last_error() == ""
    plan.close()
