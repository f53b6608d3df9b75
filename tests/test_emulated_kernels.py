"""The library's host logic and kernel bodies, run on the CPU, against the oracle.

tests/emu/libua2a_emu.so links the library's own host code (plans, argument
checks, path choice, launch geometry) with a backend that executes the
kernels' per-thread bodies for every tile and thread on the CPU (the LDS
kernel's fill phase for all threads before its drain phase).  Buffers are
host memory with guard bands around them, so an out-of-range write shows as a
changed guard byte; a second build under AddressSanitizer (run in a child
process) reports out-of-range reads and writes of the exact-size buffers.

Every output is compared byte for byte with the CPU oracle.  No GPU is used.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import ulysses_all_re_amd as ua
from tests.emu import build as emu_build
from workloads import TAIL_SHAPES

GUARD = 64
GUARD_BYTE = 0x5A

SHAPES = [
    (2, 1, 8, 4, 16, 2),       # the tiny workload's shape, bf16-sized
    (1, 2, 3, 5, 7, 2),        # w = 1
    (3, 2, 5, 6, 4, 4),
    (4, 3, 7, 8, 3, 8),
    (5, 1, 4, 10, 2, 1),
    (2, 2, 9, 4, 64, 2),       # run 128 B
    (4, 1, 40, 8, 128, 2),     # run 512 B: direct path, several tiles
    (3, 2, 33, 12, 80, 4),     # awkward-shaped, run 1280 B
    (8, 1, 13, 40, 128, 2),    # video-DiT head layout, short sequence
    (2, 1, 37, 2, 1024, 2),    # 4 KiB rows: grouped tile order in mode 0, padding tiles
    (4, 2, 13, 8, 256, 2),     # 4 KiB rows, two planes
] + [s[:5] + ({"bf16": 2, "fp16": 2, "fp32": 4, "f64": 8, "u8": 1}[s[5]],) for s in TAIL_SHAPES]


def _load(sanitize=False):
    path = emu_build.library_path(sanitize)
    srcs = emu_build.SOURCES + [os.path.join(emu_build.CSRC, h) for h in
                                ("ua2a_geometry.h", "ua2a_bodies.h", "ua2a_internal.h")]
    if not os.path.exists(path) or any(os.path.getmtime(s) > os.path.getmtime(path) for s in srcs):
        emu_build.build(sanitize)
    lib = ua.declare_signatures(ctypes.CDLL(path))
    lib.ua2a_emu_fail_next_launch.argtypes = [ctypes.c_int]
    lib.ua2a_emu_set_device.argtypes = [ctypes.c_int]
    lib.ua2a_emu_kernel_count.argtypes = [ctypes.c_int]
    lib.ua2a_emu_last_grid.restype = ctypes.c_uint
    return lib


@pytest.fixture(scope="module")
def emu():
    return _load()


class Buf:
    """Host buffer of `nbytes` whose start is `misalign` bytes past a 64-byte boundary,
    with GUARD bytes of a known pattern on both sides."""

    def __init__(self, nbytes, misalign=0):
        self.raw = np.full(nbytes + 2 * GUARD + 128, GUARD_BYTE, dtype=np.uint8)
        base = self.raw.ctypes.data
        start = (-(base + GUARD) % 64) + GUARD + misalign
        self.start, self.n = start, nbytes
        self.view = self.raw[start:start + nbytes]
        self.ptr = base + start

    def guards_intact(self):
        return bool((self.raw[:self.start] == GUARD_BYTE).all() and
                    (self.raw[self.start + self.n:] == GUARD_BYTE).all())


def rand_bytes(n, seed):
    return np.random.default_rng(seed).integers(0, 256, size=n, dtype=np.uint8)


def emu_exchange(lib, shape, mode, chunked=False, path=ua.UA2A_PATH_AUTO, in_mis=0, out_mis=0,
                 win_mis=0, seed=0, blocks=0):
    """Run one exchange through the emulated library; returns (x, out bytes, info, bufs)."""
    w, B, S, H, D, e = shape
    lay = ua2a_layout(lib, w, B, S, H, D, e)
    n = lay.tensor_bytes
    xin = Buf(n, in_mis)
    xin.view[:] = rand_bytes(n, seed)
    xout = Buf(n, out_mis)
    win = Buf(lay.window_bytes, win_mis) if chunked else None
    h = ctypes.c_void_p()
    rc = lib.ua2a_plan(ctypes.byref(h), w, B, S, H, D, e, blocks,
                       win.ptr if win else None, lay.window_bytes if win else 0, 0)
    assert rc == 0, rc
    try:
        assert lib.ua2a_plan_set_path(h, path) == 0
        info = ua.ua2a_launch_info_t()
        assert lib.ua2a_describe(h, mode, int(chunked), xin.ptr, xout.ptr, ctypes.byref(info)) == 0
        lib.ua2a_emu_reset_counts()
        rc = lib.ua2a_exchange(h, mode, int(chunked), xin.ptr, xout.ptr, None)
        assert rc == 0, (rc, lib.ua2a_plan_last_error(h))
        assert lib.ua2a_emu_launches() == info.launches
    finally:
        lib.ua2a_destroy(h)
    bufs = [xin, xout] + ([win] if win else [])
    return xin.view.copy(), xout.view.copy(), info, bufs


def ua2a_layout(lib, w, B, S, H, D, e):
    lay = ua.ua2a_layout_t()
    assert lib.ua2a_layout(w, B, S, H, D, e, ctypes.byref(lay)) == 0
    return lay


def oracle_bytes(xbytes, shape, mode, chunked=False):
    w, B, S, H, D, e = shape
    dt = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[e]
    ishape = (w, B, S, H, D) if mode == 0 else (w, B, S * w, H // w, D)
    x = xbytes.view(dt).reshape(ishape)
    return oracle.exchange(x, mode, w, chunked=chunked).view(np.uint8).ravel()


@pytest.mark.parametrize("path", [ua.UA2A_PATH_AUTO, ua.UA2A_PATH_DIRECT, ua.UA2A_PATH_LDS],
                         ids=["auto", "direct", "lds"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_emulated_matches_oracle(emu, shape, path):
    for mode in (0, 1):
        for chunked in (False, True):
            x, y, info, bufs = emu_exchange(emu, shape, mode, chunked, path, seed=mode)
            assert np.array_equal(y, oracle_bytes(x, shape, mode, chunked=False)), (mode, chunked)
            assert all(b.guards_intact() for b in bufs), (mode, chunked)
            assert bufs[0].view.tobytes() == x.tobytes()      # input untouched
            if path != ua.UA2A_PATH_AUTO:
                assert info.path == path or (path == ua.UA2A_PATH_LDS and info.lds_rows == 0)


@pytest.mark.parametrize("mis", [(2, 0, 0), (0, 4, 0), (6, 10, 2), (8, 8, 8)])
@pytest.mark.parametrize("shape", [(4, 1, 40, 8, 128, 2), (3, 1, 5, 3, 7, 2), (2, 2, 9, 4, 64, 2)],
                         ids=lambda s: "x".join(map(str, s)))
def test_emulated_misaligned_bases(emu, shape, mis):
    """Element-aligned but not 16-byte-aligned tensors and window take the narrower paths."""
    e = shape[5]
    mis = tuple(m - m % e for m in mis)
    for path in (ua.UA2A_PATH_AUTO, ua.UA2A_PATH_DIRECT, ua.UA2A_PATH_LDS):
        for mode in (0, 1):
            for chunked in (False, True):
                x, y, info, bufs = emu_exchange(emu, shape, mode, chunked, path, *mis, seed=3)
                assert np.array_equal(y, oracle_bytes(x, shape, mode)), (path, mode, chunked)
                assert all(b.guards_intact() for b in bufs)
                if mis[0] % 16 or mis[1] % 16:
                    assert info.vector_bytes < 16


@pytest.mark.parametrize("shape,mis", [((130, 1, 3, 130, 7, 2), 0), ((130, 2, 5, 260, 3, 2), 2),
                                       ((4, 1, 61, 4, 7, 2), 6)],
                         ids=["w130", "w130-B2-misaligned", "w4-odd-S"])
def test_emulated_lds_partial_chunks(emu, shape, mis):
    """A spans that start or end inside a 16-byte chunk (odd S_local * run, offset
    bases): mode 1 reads those chunks whole and places their in-span pieces; with
    w = 130 its 2w partial-chunk slots outnumber the 256 lanes of a workgroup, so
    lanes take a second slot."""
    for mode in (0, 1):
        x, y, info, bufs = emu_exchange(emu, shape, mode, path=ua.UA2A_PATH_LDS, in_mis=mis,
                                        out_mis=mis, seed=11 + mode)
        assert info.path == ua.UA2A_PATH_LDS and info.vector_bytes < 16
        assert np.array_equal(y, oracle_bytes(x, shape, mode)), mode
        assert all(b.guards_intact() for b in bufs), mode


@pytest.mark.parametrize("blocks", [1, 3, 7, 64, 100000])
def test_emulated_blocks_hint_does_not_change_bytes(emu, blocks):
    shape = (4, 1, 40, 8, 128, 2)
    ref = None
    for mode in (0, 1):
        x, y, info, _ = emu_exchange(emu, shape, mode, blocks=blocks, seed=5)
        assert np.array_equal(y, oracle_bytes(x, shape, mode))
        assert info.grid == min(blocks, info.tiles)
        ref = y if ref is None else ref


def test_emulated_round_trip_and_chunked_launch_count(emu):
    shape = (4, 4, 32, 16, 64, 2)
    w, B, S, H, D, e = shape
    x, y, info, _ = emu_exchange(emu, shape, 0, chunked=True, seed=7)
    # the whole chunked exchange is one launch of the chunked kernel
    assert info.launches == 1 and info.chunked_form == ua.UA2A_CHUNKED_ONE_LAUNCH
    assert emu.ua2a_emu_kernel_count(7) == 1 and emu.ua2a_emu_launches() == 1
    assert np.array_equal(y, oracle_bytes(x, shape, 0))
    # feed mode 0's output back through mode 1
    lay = ua2a_layout(emu, *shape)
    src, dst = Buf(lay.tensor_bytes), Buf(lay.tensor_bytes)
    src.view[:] = y
    h = ctypes.c_void_p()
    assert emu.ua2a_plan(ctypes.byref(h), w, B, S, H, D, e, 0, None, 0, 0) == 0
    assert emu.ua2a_exchange(h, 1, 0, src.ptr, dst.ptr, None) == 0
    emu.ua2a_destroy(h)
    assert dst.view.tobytes() == x.tobytes()


# ------------------------------------------------------ magic-number division

@pytest.mark.parametrize("shape", [(4, 4, 32, 16, 64, 2), (3, 3, 5, 6, 4, 4), (2, 5, 9, 4, 64, 2),
                                   (5, 2, 4, 10, 2, 1), (4, 3, 7, 8, 3, 8), (2, 3, 37, 2, 1024, 2)],
                         ids=lambda s: "x".join(map(str, s)))
def test_emulated_chunked_forms(emu, shape):
    """Every chunked exchange is one launch: of the chunked kernel on the
    direct path (its 3-D grid, the grouped order's 3-D grid for 4 KiB rows in
    mode 0, or a flat grid under a blocks hint, whose workgroups loop over
    tiles), in which every lane reads back only window bytes it stored itself
    (the emulation tracks each window byte's last writer), or of the chunked
    LDS kernel, whose lanes likewise read back only window bytes they stored
    in the same plane.  Every form matches the oracle, leaves the guard bands
    alone and ends with the last plane in the window."""
    w, B, S, H, D, e = shape
    assert (S * H * D * e) % 16 == 0
    for mode in (0, 1):
        for path, blocks in ((ua.UA2A_PATH_DIRECT, 0), (ua.UA2A_PATH_DIRECT, 5), (ua.UA2A_PATH_LDS, 0),
                             (ua.UA2A_PATH_LDS, 3)):
            x, y, info, bufs = emu_exchange(emu, shape, mode, True, path, blocks=blocks, seed=11 + mode)
            assert np.array_equal(y, oracle_bytes(x, shape, mode)), (mode, path, blocks)
            assert all(b.guards_intact() for b in bufs), (mode, path, blocks)
            lds = info.path == ua.UA2A_PATH_LDS
            assert info.chunked_form == ua.UA2A_CHUNKED_ONE_LAUNCH and info.launches == 1, (mode, path, blocks)
            assert emu.ua2a_emu_kernel_count(7) == (0 if lds else 1)
            assert emu.ua2a_emu_kernel_count(9) == (1 if lds else 0)
            assert emu.ua2a_emu_kernel_count(2) == 0
            assert info.grid_dims == (1 if lds or blocks else 3), (mode, path, blocks)
            if blocks:
                assert 1 <= info.grid <= blocks, (mode, path, blocks)
            # the window holds the last plane of every rank, in the output's layout
            out = y.reshape(w, B, -1)
            assert np.array_equal(bufs[2].view.reshape(w, -1), out[:, B - 1]), (mode, path, blocks)


@pytest.mark.parametrize("mis", [0, 8, 4, 2], ids=lambda m: f"mis{m}")
@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 7, 9])
def test_emulated_chunked_one_launch_planes(emu, B, mis):
    """The one-launch chunked kernel over 1-9 planes with 16-, 8-, 4- and
    2-byte vectors (bases misaligned to match), so every count of planes in
    flight per lane meets a remainder; output, guards and window checked."""
    shape = (4, B, 6, 8, 32, 2)      # run 128 B, slabs of 768 B: partial tiles
    w = shape[0]
    for mode in (0, 1):
        x, y, info, bufs = emu_exchange(emu, shape, mode, True, ua.UA2A_PATH_DIRECT, mis, mis, mis,
                                        seed=31 + B + mode)
        assert info.chunked_form == ua.UA2A_CHUNKED_ONE_LAUNCH and info.launches == 1
        assert info.vector_bytes == (16 if mis == 0 else mis)
        assert np.array_equal(y, oracle_bytes(x, shape, mode)), mode
        assert all(b.guards_intact() for b in bufs), mode
        assert np.array_equal(bufs[2].view.reshape(w, -1), y.reshape(w, B, -1)[:, B - 1]), mode


@pytest.mark.parametrize("shape,mis", [
    ((3, 4, 8, 3, 7, 2), (0, 0, 0)),          # run 14 B: 2-byte pieces
    ((3, 4, 8, 3, 7, 2), (2, 2, 2)),          # ... spans off the 16-byte grid: partial chunks
    ((4, 3, 64, 4, 7, 2), (6, 6, 6)),         # line-aligned tiles, bases 6 bytes off
    ((2, 5, 4, 6, 5, 4), (4, 4, 4)),          # run 60 B, 4-byte pieces
    ((2, 3, 80, 2, 12, 2), (0, 0, 0)),        # run 24 B, spans of whole chunks
    ((8, 2, 257, 8, 24, 2), (8, 8, 8)),       # run 48 B, 8-byte pieces, odd S_local
    ((2, 9, 300, 4, 16, 2), (0, 0, 0)),       # run 64 B, 16-byte pieces, nine planes
    ((3, 2, 16, 3, 5, 1), (3, 3, 3)),         # run 5 B: 1-byte pieces
    ((130, 2, 8, 260, 3, 2), (2, 2, 2)),      # 2w partial-chunk slots > 256 lanes
    ((3, 2, 16, 3, 5, 1), (0, 5, 5)),         # input off by 5, output and window agree
    ((1, 3, 8, 4, 7, 2), (0, 2, 2)),          # w = 1: one head block, window = one plane
    ((3, 4, 8, 3, 7, 2), (0, 0, 2)),          # window 2 bytes off the output: pieces out
    ((3, 4, 8, 3, 7, 2), (0, 4, 0)),          # output 4 bytes off the window: pieces out
    ((3, 3, 7, 3, 7, 2), (0, 0, 0)),          # plane 294 B: the output's offset moves per plane
    ((4, 3, 61, 4, 7, 2), (6, 6, 6)),         # plane 3416 B, bases 6 bytes off
    ((5, 2, 37, 10, 3, 1), (3, 3, 3)),        # plane 1110 B, 1-byte pieces
    ((2, 5, 3, 6, 5, 4), (4, 8, 12)),         # run 60 B, plane 360 B, three different offsets
], ids=lambda v: "x".join(map(str, v)))
def test_emulated_chunked_lds_one_launch(emu, shape, mis):
    """The LDS path's chunked exchange is one launch of the chunked LDS
    kernel whatever the bases' offsets and the plane size: window chunks go to
    the output as whole 16-byte stores where the output lies at the window's
    offset modulo 16, else as pieces.  LDS holds two planes at once when a
    plane is a multiple of 16 bytes (one otherwise, and at the end of an odd
    count).  It matches the oracle, keeps the guard bands and ends with the
    last plane in the window; the emulation checks that each lane reads back
    only window bytes that it stored in the same plane, and that every window
    byte is written."""
    w, B, S, H, D, e = shape
    plane = S * H * D * e
    for mode in (0, 1):
        x, y, info, bufs = emu_exchange(emu, shape, mode, True, ua.UA2A_PATH_LDS, *mis, seed=41 + B + mode)
        assert info.path == ua.UA2A_PATH_LDS, mode
        assert info.chunked_form == ua.UA2A_CHUNKED_ONE_LAUNCH and info.launches == 1, mode
        assert info.lds_planes == (min(B, 2) if plane % 16 == 0 else 1), mode
        assert info.lds_bytes % 16 == 0 and info.lds_bytes <= 65536, mode
        assert emu.ua2a_emu_kernel_count(9) == 1 and emu.ua2a_emu_kernel_count(2) == 0, mode
        assert np.array_equal(y, oracle_bytes(x, shape, mode)), mode
        assert all(b.guards_intact() for b in bufs), mode
        assert np.array_equal(bufs[2].view.reshape(w, -1), y.reshape(w, B, -1)[:, B - 1]), mode


def test_emulated_chunked_many_planes(emu):
    """Forty planes through one window, in one launch; the result the oracle's."""
    shape = (3, 40, 5, 6, 8, 2)
    w, B, S, H, D, e = shape
    for mode in (0, 1):
        x, y, info, bufs = emu_exchange(emu, shape, mode, True, ua.UA2A_PATH_DIRECT, seed=17 + mode)
        assert info.launches == 1 and emu.ua2a_emu_kernel_count(7) == 1
        assert np.array_equal(y, oracle_bytes(x, shape, mode)), mode
        assert all(b.guards_intact() for b in bufs), mode


def test_fdiv_matches_exact_division(emu):
    """The kernels' multiply-high division against exact integer division."""
    fn = emu.ua2a_emu_fdiv
    fn.argtypes = [ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    rng = np.random.default_rng(5)
    top = 2 ** 32 - 1
    divisors = ([1, 2, 3, 5, 7, 10, 14, 40, 80, 96, 640, 1000, 2 ** 16 - 1, 2 ** 16, 2 ** 16 + 1,
                 2 ** 31 - 1, 2 ** 31, 2 ** 31 + 1, top - 1, top] +
                [1 << k for k in range(32)] + rng.integers(1, top, 300, dtype=np.uint64).tolist())
    n = np.concatenate([np.arange(0, 4096), top - np.arange(0, 4096),
                        rng.integers(0, top, 20000, dtype=np.uint64)]).astype(np.uint32)
    q = np.empty_like(n)
    for d in divisors:
        edges = np.array([d - 1, d, d + 1, 2 * d - 1, 2 * d, (top // d) * d, (top // d) * d - 1],
                         dtype=np.uint64)
        nn = np.concatenate([n, np.clip(edges, 0, top).astype(np.uint32)])
        qq = np.empty_like(nn)
        fn(int(d), nn.ctypes.data, qq.ctypes.data, nn.size)
        assert np.array_equal(qq, (nn.astype(np.uint64) // np.uint64(d)).astype(np.uint32)), d


# ------------------------------------------------------------- error handling

def _plan(lib, shape=(2, 2, 4, 4, 8, 2), window=None, wbytes=0, device=0):
    w, B, S, H, D, e = shape
    h = ctypes.c_void_p()
    rc = lib.ua2a_plan(ctypes.byref(h), w, B, S, H, D, e, 0, window, wbytes, device)
    return rc, h


def test_lds_slot_order_visits_every_tile_once(emu):
    """The LDS kernels deal tiles to the XCDs in runs of 2^xlog consecutive tiles:
    launch slot L -> tile.  Over num_slots = num_tiles rounded up to 8 * 2^xlog
    slots (as the host launches them) every tile runs exactly once, the rest of
    the slots are empty, and the 8 slots of one XCD turn hold consecutive runs."""
    fn = emu.ua2a_emu_lds_slot_tiles
    fn.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
    for xlog in range(5):
        span = 8 << xlog
        for num_tiles in list(range(1, 70)) + [255, 256, 257, 1000, 4681 * 4, 65537]:
            slots = -(-num_tiles // span) * span
            out = np.zeros(slots, dtype=np.uint32)
            fn(slots, xlog, out.ctypes.data)
            used = np.sort(out[out < num_tiles])
            assert np.array_equal(used, np.arange(num_tiles)), (xlog, num_tiles)
            assert np.array_equal(np.sort(out), np.arange(slots)), (xlog, num_tiles)
            # slots L and L + 8 run on the same XCD: consecutive tiles within a run
            run = 1 << xlog
            for L in range(0, min(slots, 4 * span)):
                if (L // 8) % run != run - 1:
                    assert out[L + 8] == out[L] + 1, (xlog, num_tiles, L)


def test_layout_and_plan_errors(emu):
    lay = ua.ua2a_layout_t()
    assert emu.ua2a_layout(2, 1, 8, 4, 16, 2, None) == ua.UA2A_ERR_INVALID_ARG
    assert emu.ua2a_layout(2, 1, 8, 4, 16, 3, ctypes.byref(lay)) == ua.UA2A_ERR_INVALID_ARG
    assert emu.ua2a_layout(2, 1, 8, 3, 16, 2, ctypes.byref(lay)) == ua.UA2A_ERR_SHAPE
    for bad in [(0, 1, 8, 4, 16), (2, 0, 8, 4, 16), (2, 1, 0, 4, 16), (2, 1, 8, 0, 16),
                (2, 1, 8, 4, 0), (2, 1, 2 ** 31, 4, 16), (2, 1, 8, 2 ** 20, 2 ** 20),
                (65537, 1, 1, 65537, 1), (256, 1, 2 ** 30, 256, 1)]:
        assert emu.ua2a_layout(*bad, 2, ctypes.byref(lay)) == ua.UA2A_ERR_SHAPE, bad
    assert emu.ua2a_layout(8, 1, 9450, 40, 128, 2, ctypes.byref(lay)) == 0
    assert (lay.H_local, lay.S_global, lay.run_bytes) == (5, 75600, 1280)
    assert lay.tensor_bytes == 774144000 and lay.moved_bytes == 2 * 774144000
    assert lay.window_bytes == 8 * 9450 * 40 * 128 * 2
    h = ctypes.c_void_p()
    assert emu.ua2a_plan(None, 2, 1, 8, 4, 16, 2, 0, None, 0, 0) == ua.UA2A_ERR_INVALID_ARG
    assert emu.ua2a_plan(ctypes.byref(h), 2, 1, 8, 4, 16, 2, -1, None, 0, 0) == ua.UA2A_ERR_INVALID_ARG
    assert emu.ua2a_plan(ctypes.byref(h), 2, 1, 8, 4, 16, 2, 0, None, 16, 0) == ua.UA2A_ERR_INVALID_ARG
    assert emu.ua2a_plan(ctypes.byref(h), 2, 1, 8, 4, 16, 2, 0, None, 0, -1) == ua.UA2A_ERR_INVALID_ARG
    buf = Buf(4096, 1)
    assert emu.ua2a_plan(ctypes.byref(h), 2, 1, 8, 4, 16, 2, 0, buf.ptr, 4096, 0) == ua.UA2A_ERR_ALIGN
    assert h.value is None
    for code in range(-9, 1):
        assert emu.ua2a_status_string(code)
    assert emu.ua2a_status_string(-100) == b"unknown status"


def test_exchange_argument_errors(emu):
    shape = (2, 2, 4, 4, 8, 2)
    lay = ua2a_layout(emu, *shape)
    n = lay.tensor_bytes
    a, b = Buf(n), Buf(n)
    rc, h = _plan(emu, shape)
    assert rc == 0
    assert emu.ua2a_exchange(None, 0, 0, a.ptr, b.ptr, None) == ua.UA2A_ERR_INVALID_ARG
    assert emu.ua2a_exchange(h, 2, 0, a.ptr, b.ptr, None) == ua.UA2A_ERR_INVALID_ARG
    assert emu.ua2a_exchange(h, 0, 2, a.ptr, b.ptr, None) == ua.UA2A_ERR_INVALID_ARG
    assert emu.ua2a_exchange(h, 0, 0, None, b.ptr, None) == ua.UA2A_ERR_INVALID_ARG
    assert emu.ua2a_exchange(h, 0, 0, a.ptr + 1, b.ptr, None) == ua.UA2A_ERR_ALIGN
    assert emu.ua2a_exchange(h, 0, 0, a.ptr, a.ptr, None) == ua.UA2A_ERR_ALIAS
    big = Buf(2 * n)
    # partial overlap with different pointers is still rejected (byte ranges)
    assert emu.ua2a_exchange(h, 0, 0, big.ptr, big.ptr + n - 2, None) == ua.UA2A_ERR_ALIAS
    assert emu.ua2a_exchange(h, 1, 0, big.ptr + n - 2, big.ptr, None) == ua.UA2A_ERR_ALIAS
    assert emu.ua2a_exchange(h, 0, 0, big.ptr, big.ptr + n, None) == 0      # adjacent is fine
    assert emu.ua2a_exchange(h, 0, 1, a.ptr, b.ptr, None) == ua.UA2A_ERR_CAPACITY
    emu.ua2a_destroy(h)
    small = Buf(lay.window_bytes - 2)
    rc, h = _plan(emu, shape, small.ptr, lay.window_bytes - 2)
    assert emu.ua2a_exchange(h, 0, 1, a.ptr, b.ptr, None) == ua.UA2A_ERR_CAPACITY
    assert emu.ua2a_exchange(h, 0, 0, a.ptr, b.ptr, None) == 0    # unchunked needs no window
    emu.ua2a_destroy(h)
    rc, h = _plan(emu, shape, big.ptr + 2, lay.window_bytes)      # window inside `out`
    assert emu.ua2a_exchange(h, 0, 1, a.ptr, big.ptr, None) == ua.UA2A_ERR_ALIAS
    emu.ua2a_destroy(h)
    info = ua.ua2a_launch_info_t()
    rc, h = _plan(emu, shape)
    assert emu.ua2a_describe(h, 0, 0, a.ptr, b.ptr, None) == ua.UA2A_ERR_INVALID_ARG
    assert emu.ua2a_describe(h, 0, 0, a.ptr, a.ptr, ctypes.byref(info)) == ua.UA2A_ERR_ALIAS
    assert emu.ua2a_plan_set_path(h, 3) == ua.UA2A_ERR_INVALID_ARG
    assert emu.ua2a_plan_last_error(h) == b""
    emu.ua2a_destroy(h)


def test_device_mismatch_and_sticky_disable(emu):
    shape = (2, 2, 4, 4, 8, 2)
    lay = ua2a_layout(emu, *shape)
    a, b = Buf(lay.tensor_bytes), Buf(lay.tensor_bytes)
    rc, h = _plan(emu, shape, device=1)
    assert emu.ua2a_exchange(h, 0, 0, a.ptr, b.ptr, None) == ua.UA2A_ERR_DEVICE
    emu.ua2a_emu_set_device(1)
    try:
        assert emu.ua2a_exchange(h, 0, 0, a.ptr, b.ptr, None) == 0
        # a failed launch disables the plan for good, with a reason
        emu.ua2a_emu_fail_next_launch(98)
        assert emu.ua2a_exchange(h, 0, 0, a.ptr, b.ptr, None) == ua.UA2A_ERR_HIP
        assert b"failed" in emu.ua2a_plan_last_error(h)
        assert emu.ua2a_exchange(h, 0, 0, a.ptr, b.ptr, None) == ua.UA2A_ERR_DISABLED
        assert emu.ua2a_exchange(h, 1, 0, a.ptr, b.ptr, None) == ua.UA2A_ERR_DISABLED
        info = ua.ua2a_launch_info_t()
        assert emu.ua2a_describe(h, 0, 0, a.ptr, b.ptr, ctypes.byref(info)) == ua.UA2A_ERR_DISABLED
    finally:
        emu.ua2a_emu_set_device(0)
    assert emu.ua2a_destroy(h) == 0           # consumes a disabled plan
    assert emu.ua2a_destroy(None) == 0


def test_chunked_failure_mid_plane_disables(emu):
    shape = (2, 3, 4, 4, 8, 2)
    lay = ua2a_layout(emu, *shape)
    a, b, win = Buf(lay.tensor_bytes), Buf(lay.tensor_bytes), Buf(lay.window_bytes)
    rc, h = _plan(emu, shape, win.ptr, lay.window_bytes)
    emu.ua2a_emu_fail_next_launch(7)
    assert emu.ua2a_exchange(h, 0, 1, a.ptr, b.ptr, None) == ua.UA2A_ERR_HIP
    assert emu.ua2a_exchange(h, 0, 1, a.ptr, b.ptr, None) == ua.UA2A_ERR_DISABLED
    emu.ua2a_destroy(h)


def test_grouped_tile_order_covers_every_vector(emu):
    """Mode 0 on 4 KiB-multiple rows uses the interleaved order; padding tiles stay empty."""
    shape = (2, 3, 37, 2, 1024, 2)        # row 4096 B, 74 tiles per slab, groups of 8
    for mode in (0, 1):
        x, y, info, bufs = emu_exchange(emu, shape, mode, seed=9)
        assert np.array_equal(y, oracle_bytes(x, shape, mode))
        assert all(b.guards_intact() for b in bufs)
    w, B, S = shape[:3]
    slabs, tps = w * B * w, -(-S * 128 // 64)
    lay = ua2a_layout(emu, *shape)
    a, b = Buf(lay.tensor_bytes), Buf(lay.tensor_bytes)
    rc, h = _plan(emu, shape)
    info = ua.ua2a_launch_info_t()
    assert emu.ua2a_describe(h, 0, 0, a.ptr, b.ptr, ctypes.byref(info)) == 0
    assert info.tiles == slabs * -(-tps // 8) * 8          # padded to whole groups
    assert emu.ua2a_describe(h, 1, 0, a.ptr, b.ptr, ctypes.byref(info)) == 0
    assert info.tiles == w * B * -(-S * 2 * 128 // 64)       # mode 1: slab after slab
    emu.ua2a_destroy(h)


def test_path_choice(emu):
    def describe(shape, mis=0, path=ua.UA2A_PATH_AUTO):
        w, B, S, H, D, e = shape
        lay = ua2a_layout(emu, *shape)
        a, b = Buf(lay.tensor_bytes, mis), Buf(lay.tensor_bytes)
        rc, h = _plan(emu, shape)
        emu.ua2a_plan_set_path(h, path)
        info = ua.ua2a_launch_info_t()
        assert emu.ua2a_describe(h, 0, 0, a.ptr, b.ptr, ctypes.byref(info)) == 0
        emu.ua2a_destroy(h)
        return info
    big = describe((8, 1, 9450, 40, 128, 2))       # video-DiT: run 1280 B
    assert (big.path, big.vector_bytes, big.launches) == (ua.UA2A_PATH_DIRECT, 16, 1)
    short = describe((2, 1, 8, 4, 16, 2))          # run 64 B
    assert (short.path, short.vector_bytes) == (ua.UA2A_PATH_LDS, 16)
    odd = describe((3, 1, 5, 3, 7, 2))             # run 14 B
    assert (odd.path, odd.vector_bytes) == (ua.UA2A_PATH_LDS, 2)
    assert describe((8, 1, 9450, 40, 128, 2), mis=2).vector_bytes == 2
    huge_row = describe((2, 1, 4, 2, 8192, 4), path=ua.UA2A_PATH_LDS)   # row > LDS tile
    assert huge_row.path == ua.UA2A_PATH_DIRECT and huge_row.lds_rows == 0


# ----------------------------------------------------------- sanitizer build

ASAN_DRIVER = r"""
import ctypes, sys
import numpy as np
sys.path.insert(0, {root!r})
import oracle, ulysses_all_re_amd as ua
lib = ua.declare_signatures(ctypes.CDLL({lib!r}))
cases = {cases!r}
for (w, B, S, H, D, e, mode, chunked, path, mis, blocks) in cases:
    lay = ua.ua2a_layout_t()
    assert lib.ua2a_layout(w, B, S, H, D, e, ctypes.byref(lay)) == 0
    n = lay.tensor_bytes
    # exact-size heap blocks (plus the misalignment), so ASan sees any overrun
    xin = (ctypes.c_uint8 * (n + mis))()
    xout = (ctypes.c_uint8 * (n + mis))()
    win = (ctypes.c_uint8 * (lay.window_bytes + mis))() if chunked else None
    src = np.frombuffer(xin, dtype=np.uint8)[mis:]
    src[:] = np.random.default_rng(w * 131 + S).integers(0, 256, n, dtype=np.uint8)
    h = ctypes.c_void_p()
    assert lib.ua2a_plan(ctypes.byref(h), w, B, S, H, D, e, blocks,
                         (ctypes.addressof(win) + mis) if chunked else None,
                         lay.window_bytes if chunked else 0, 0) == 0
    assert lib.ua2a_plan_set_path(h, path) == 0
    rc = lib.ua2a_exchange(h, mode, chunked, ctypes.addressof(xin) + mis, ctypes.addressof(xout) + mis, None)
    assert rc == 0, rc
    lib.ua2a_destroy(h)
    dt = {{1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}}[e]
    ishape = (w, B, S, H, D) if mode == 0 else (w, B, S * w, H // w, D)
    want = oracle.exchange(src.view(dt).reshape(ishape), mode, w).view(np.uint8).ravel()
    got = np.frombuffer(xout, dtype=np.uint8)[mis:]
    assert np.array_equal(got, want), (w, B, S, H, D, e, mode, chunked, path, mis, blocks)
print("asan-ok", len(cases))
"""


@pytest.mark.slow
def test_emulated_kernels_under_asan(tmp_path):
    lib = emu_build.build(sanitize=True)
    cases = []
    for shape in SHAPES:
        for mode in (0, 1):
            for chunked in (0, 1):
                for path in (ua.UA2A_PATH_DIRECT, ua.UA2A_PATH_LDS):
                    cases.append((*shape, mode, chunked, path, 0, 0))
    for shape in [(3, 1, 5, 3, 7, 2), (4, 1, 40, 8, 128, 2), (2, 2, 9, 4, 64, 2)]:
        for mode in (0, 1):
            for path in (ua.UA2A_PATH_DIRECT, ua.UA2A_PATH_LDS):
                cases.append((*shape, mode, 1, path, 2, 0))
    for mode in (0, 1):      # more partial-chunk slots than lanes
        cases.append((130, 2, 5, 260, 3, 2, mode, 0, ua.UA2A_PATH_LDS, 2, 0))
    # the LDS path's one-launch chunked kernel: partial chunks, several planes, a capped grid,
    # planes that are not whole 16-byte chunks
    for shape in [(4, 3, 64, 4, 7, 2), (130, 2, 8, 260, 3, 2), (2, 5, 4, 6, 5, 4), (8, 2, 257, 8, 24, 2),
                  (3, 2, 16, 3, 5, 1), (3, 3, 7, 3, 7, 2), (4, 3, 61, 4, 7, 2)]:
        for mode in (0, 1):
            for mis, blocks in ((0, 0), (2, 0), (0, 5)):
                cases.append((*shape, mode, 1, ua.UA2A_PATH_LDS, mis - mis % shape[5], blocks))
    # capped flat grids: groups of four tiles per workgroup, partial groups, remainders
    for shape in [(4, 3, 50, 8, 16, 2), (3, 2, 33, 12, 80, 4), (2, 2, 37, 2, 1024, 2)]:
        for mode in (0, 1):
            for chunked in (0, 1):
                for blocks in (3, 7):
                    cases.append((*shape, mode, chunked, ua.UA2A_PATH_DIRECT, 0, blocks))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = tmp_path / "asan_driver.py"
    script.write_text(ASAN_DRIVER.format(root=root, lib=lib, cases=cases))
    env = dict(os.environ, LD_PRELOAD=emu_build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, str(script)], env=env, capture_output=True, text=True,
                         timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-6000:]
    assert "asan-ok" in res.stdout


# ------------------------------------------------------- property-based sweep

from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402


@st.composite
def exchange_cases(draw):
    w = draw(st.integers(1, 6))
    hl = draw(st.integers(1, 5))
    e = draw(st.sampled_from([1, 2, 4, 8]))
    B = draw(st.integers(1, 3))
    S = draw(st.integers(1, 40))
    D = draw(st.integers(1, 48))
    mode = draw(st.integers(0, 1))
    chunked = draw(st.booleans())
    path = draw(st.sampled_from([ua.UA2A_PATH_AUTO, ua.UA2A_PATH_DIRECT, ua.UA2A_PATH_LDS]))
    mis = tuple(draw(st.integers(0, 15)) // e * e for _ in range(3))
    blocks = draw(st.sampled_from([0, 1, 3, 1000]))
    return (w, B, S, w * hl, D, e), mode, chunked, path, mis, blocks


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(case=exchange_cases())
def test_emulated_random_cases_match_oracle(emu, case):
    shape, mode, chunked, path, mis, blocks = case
    x, y, info, bufs = emu_exchange(emu, shape, mode, chunked, path, *mis, seed=sum(shape),
                                    blocks=blocks)
    assert np.array_equal(y, oracle_bytes(x, shape, mode)), (case, info.path, info.vector_bytes)
    assert all(b.guards_intact() for b in bufs), case
