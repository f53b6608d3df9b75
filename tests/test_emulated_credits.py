"""Readiness credits (ua2a_exchange_publish, ua2a_wait_credits) on the host emulation.

The publishing exchange must (i) produce the oracle's bytes, (ii) add exactly
1 to every receiving rank's counter per call, whatever the number of parts,
grid or vector width, and (iii) never credit a receiver before all of its
bytes are stored: when the emulated stream stops part-way (the emulator's
tile budget; later launches on the stream then never start, as in stream
order), every receiver already credited holds the oracle's bytes.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import ulysses_all_re_amd as ua
from tests.test_emulated_kernels import Buf, _load, oracle_bytes, rand_bytes

SHAPES = [
    (2, 1, 8, 4, 16, 2),       # 64 B runs: the auto path would stage through LDS
    (3, 2, 5, 6, 4, 4),
    (4, 1, 40, 8, 128, 2),
    (3, 2, 33, 12, 80, 4),
    (8, 1, 13, 40, 128, 2),
    (2, 1, 37, 2, 1024, 2),    # 4 KiB rows: the grouped tile order is not used by parts
    (3, 1, 5, 3, 7, 2),        # 14 B runs, 2-byte vectors
    (5, 2, 7, 10, 3, 8),
]


@pytest.fixture(scope="module")
def emu():
    lib = _load()
    lib.ua2a_emu_set_tile_budget.argtypes = [ctypes.c_longlong]
    return lib


def _plan(lib, shape, blocks=0):
    w, B, S, H, D, e = shape
    h = ctypes.c_void_p()
    assert lib.ua2a_plan(ctypes.byref(h), w, B, S, H, D, e, blocks, None, 0, 0) == 0
    return h


def _run(lib, shape, mode, parts, blocks=0, calls=1, budget=-1, seed=0):
    w, B, S, H, D, e = shape
    lay = ua.ua2a_layout_t()
    assert lib.ua2a_layout(w, B, S, H, D, e, ctypes.byref(lay)) == 0
    n = lay.tensor_bytes
    xin, xout = Buf(n), Buf(n)
    xin.view[:] = rand_bytes(n, seed)
    xout.view[:] = 0xEE
    credits = np.zeros(w, dtype=np.uint32)
    h = _plan(lib, shape, blocks)
    try:
        for _ in range(calls):
            lib.ua2a_emu_reset_counts()
            lib.ua2a_emu_set_tile_budget(budget)
            try:
                rc = lib.ua2a_exchange_publish(h, mode, xin.ptr, xout.ptr, credits.ctypes.data,
                                               parts, None)
            finally:
                lib.ua2a_emu_set_tile_budget(-1)
            assert rc == 0, rc
            assert lib.ua2a_emu_kernel_count(0) == parts and lib.ua2a_emu_kernel_count(5) == 1
    finally:
        lib.ua2a_destroy(h)
    assert xin.guards_intact() and xout.guards_intact()
    return xin.view.copy(), xout.view.copy(), credits


def _parts(w):
    return sorted({1, 2, w} & set(range(1, w + 1)))


@pytest.mark.parametrize("blocks", [0, 3])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_publish_matches_oracle_and_credits_every_receiver(emu, shape, blocks):
    for mode in (0, 1):
        for parts in _parts(shape[0]):
            x, y, credits = _run(emu, shape, mode, parts, blocks=blocks, calls=2, seed=mode)
            assert np.array_equal(y, oracle_bytes(x, shape, mode)), (mode, parts)
            assert (credits == 2).all(), (mode, parts, credits)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_credited_receivers_are_complete(emu, shape):
    """Streams stopped after n tiles: each receiver already credited holds
    the oracle's bytes, and the last receiver is not credited yet."""
    w = shape[0]
    for mode in (0, 1):
        for blocks in (0, 5):
            total = _total_tiles(emu, shape, mode, blocks)
            for budget in sorted({1, total // 3, total // 2, total - 1} - {0}):
                x, y, credits = _run(emu, shape, mode, w, blocks=blocks, budget=budget, seed=7)
                want = oracle_bytes(x, shape, mode).reshape(w, -1)
                got = y.reshape(w, -1)
                assert set(np.unique(credits)) <= {0, 1} and credits[-1] == 0, (mode, budget, credits)
                for r in np.nonzero(credits == 1)[0]:
                    assert np.array_equal(got[r], want[r]), (mode, blocks, budget, r)


def _total_tiles(lib, shape, mode, blocks):
    """Tiles of a whole publishing exchange (parts = w), from the launches' descriptions."""
    w, B, S, H, D, e = shape
    run = H // w * D * e
    slab = S * run * (1 if mode == 0 else w)
    return w * B * (w if mode == 0 else 1) * -(-slab // 1024)


def test_wait_reports_unmet_targets(emu):
    credits = np.array([5, 7, 7, 0xFFFFFFFF, 1], dtype=np.uint32)
    status = np.zeros(1, dtype=np.int32)
    w = lambda first, count, target, spin=10: emu.ua2a_wait_credits(
        credits.ctypes.data, first, count, target, spin, status.ctypes.data, None)
    assert w(0, 3, 5) == 0 and status[0] == 0
    assert w(1, 2, 7) == 0 and status[0] == 0
    assert w(0, 3, 6) == 0 and status[0] == 1          # credits[0] = 5 < 6
    status[0] = 0
    assert w(3, 1, 0xFFFFFFFE) == 0 and status[0] == 0
    assert w(4, 1, 0xFFFFFFFE) == 0 and status[0] == 0  # counter wrapped past the target
    assert w(3, 1, 2) == 0 and status[0] == 1          # 3 increments short, modulo 2^32
    status[0] = 0
    assert w(0, 1, 0x80000005) == 0 and status[0] == 1


def test_credit_argument_errors(emu):
    lib = emu
    shape = (2, 1, 8, 4, 16, 2)
    n = 2 * 8 * 4 * 16 * 2
    big = Buf(4 * n)
    x, y, c = big.ptr, big.ptr + n, big.ptr + 2 * n
    h = _plan(lib, shape)
    try:
        p = lambda mode, i, o, cr, parts=2: lib.ua2a_exchange_publish(h, mode, i, o, cr, parts, None)
        assert p(0, x, y, c) == 0
        assert p(0, x, y, c, 1) == 0
        assert p(0, x, y, c, 0) == ua.UA2A_ERR_INVALID_ARG
        assert p(0, x, y, c, 3) == ua.UA2A_ERR_INVALID_ARG         # more parts than ranks
        assert p(0, x, y, None) == ua.UA2A_ERR_INVALID_ARG
        assert p(0, x, y, c + 2) == ua.UA2A_ERR_ALIGN
        assert p(0, x, y, y + 8) == ua.UA2A_ERR_ALIAS              # counters inside out
        assert p(0, x, y, x) == ua.UA2A_ERR_ALIAS                  # ... inside in
        assert p(0, x, y, y - 4) == ua.UA2A_ERR_ALIAS              # ... straddling out's start
        assert p(2, x, y, c) == ua.UA2A_ERR_INVALID_ARG
        assert p(0, x, x + 2, c) == ua.UA2A_ERR_ALIAS
        lib.ua2a_emu_set_device(1)
        assert p(0, x, y, c) == ua.UA2A_ERR_DEVICE
        lib.ua2a_emu_set_device(0)
        lib.ua2a_emu_fail_next_launch(97)
        assert p(0, x, y, c) == ua.UA2A_ERR_HIP
        assert b"publishing" in lib.ua2a_plan_last_error(h)
        assert p(0, x, y, c) == ua.UA2A_ERR_DISABLED
    finally:
        lib.ua2a_emu_set_device(0)
        lib.ua2a_destroy(h)
    s = c + 64
    wc = lambda cr, first, count, spin, st: lib.ua2a_wait_credits(cr, first, count, 0, spin, st, None)
    assert wc(c, 0, 4, 1, s) == 0
    assert wc(None, 0, 4, 1, s) == ua.UA2A_ERR_INVALID_ARG
    assert wc(c, 0, 4, 1, None) == ua.UA2A_ERR_INVALID_ARG
    assert wc(c, 0, 0, 1, s) == ua.UA2A_ERR_INVALID_ARG
    assert wc(c, -1, 4, 1, s) == ua.UA2A_ERR_INVALID_ARG
    assert wc(c, 0, 4, 0, s) == ua.UA2A_ERR_INVALID_ARG           # spin_limit 0
    assert wc(c, 2 ** 32 - 2, 4, 1, s) == ua.UA2A_ERR_INVALID_ARG
    assert wc(c, 2 ** 63 - 1, 4, 1, s) == ua.UA2A_ERR_INVALID_ARG     # first + count overflows
    assert wc(c, 0, 2 ** 32, 1, s) == ua.UA2A_ERR_INVALID_ARG
    assert wc(c + 1, 0, 4, 1, s) == ua.UA2A_ERR_ALIGN
    assert wc(c, 0, 4, 1, s + 2) == ua.UA2A_ERR_ALIGN
    assert wc(c, 0, 4, 1, c + 8) == ua.UA2A_ERR_ALIAS              # status among the counters
    lib.ua2a_emu_fail_next_launch(96)
    assert wc(c, 0, 4, 1, s) == ua.UA2A_ERR_HIP


# ----------------------------------------------------------- sanitizer build

ASAN_PUBLISH_DRIVER = r"""
import ctypes, sys
import numpy as np
sys.path.insert(0, {root!r})
import oracle, ulysses_all_re_amd as ua
lib = ua.declare_signatures(ctypes.CDLL({lib!r}))
DT = {{1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}}
for (w, B, S, H, D, e, mode, parts, blocks) in {cases!r}:
    lay = ua.ua2a_layout_t()
    assert lib.ua2a_layout(w, B, S, H, D, e, ctypes.byref(lay)) == 0
    n = lay.tensor_bytes
    xin = (ctypes.c_uint8 * n)()          # exact-size heap blocks
    xout = (ctypes.c_uint8 * n)()
    credits = (ctypes.c_uint32 * w)()
    src = np.frombuffer(xin, dtype=np.uint8)
    src[:] = np.random.default_rng(w * 7 + S).integers(0, 256, n, dtype=np.uint8)
    h = ctypes.c_void_p()
    assert lib.ua2a_plan(ctypes.byref(h), w, B, S, H, D, e, blocks, None, 0, 0) == 0
    rc = lib.ua2a_exchange_publish(h, mode, ctypes.addressof(xin), ctypes.addressof(xout),
                                   ctypes.addressof(credits), parts, None)
    assert rc == 0, rc
    lib.ua2a_destroy(h)
    ishape = (w, B, S, H, D) if mode == 0 else (w, B, S * w, H // w, D)
    want = oracle.exchange(src.view(DT[e]).reshape(ishape), mode, w).view(np.uint8).ravel()
    assert np.array_equal(np.frombuffer(xout, dtype=np.uint8), want), (w, B, S, H, D, e, mode, parts, blocks)
    assert list(credits) == [1] * w, list(credits)
print("asan-ok")
"""


@pytest.mark.slow
def test_publish_under_asan(tmp_path):
    import os
    import subprocess
    import sys

    from tests.emu import build as emu_build
    lib = emu_build.build(sanitize=True)
    cases = []
    for shape in SHAPES:
        for mode in (0, 1):
            for parts in _parts(shape[0]):
                for blocks in (0, 3):
                    cases.append((*shape, mode, parts, blocks))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = tmp_path / "asan_publish_driver.py"
    script.write_text(ASAN_PUBLISH_DRIVER.format(root=root, lib=lib, cases=cases))
    env = dict(os.environ, LD_PRELOAD=emu_build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, str(script)], env=env, capture_output=True, text=True,
                         timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-6000:]
    assert "asan-ok" in res.stdout
