"""The per-rank exchange (ua2a_exchange_ranks), run on the CPU, against the oracle.

Same host emulation as test_emulated_kernels.py: the library's own host code
with a backend that runs the per-rank kernel's body for every workgroup of the
launch grid, every loop iteration and every lane.  Each rank's tensors are
separate guarded host buffers; outputs start filled with a known byte so
that untouched runs (those of non-sending ranks) can be checked too.
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
from tests.test_emulated_kernels import SHAPES, Buf, _load, rand_bytes

FILL = 0xC3
DT = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}


@pytest.fixture(scope="module")
def emu():
    return _load()


def _layout(lib, shape):
    w, B, S, H, D, e = shape
    lay = ua.ua2a_layout_t()
    assert lib.ua2a_layout(w, B, S, H, D, e, ctypes.byref(lay)) == 0
    return lay


def _tab(ptrs):
    return (ctypes.c_void_p * len(ptrs))(*[p or None for p in ptrs])


def emu_ranks(lib, shape, mode, first, count, in_mis=None, out_mis=None, seed=0, blocks=0,
              senders_only=False):
    """One per-rank exchange through the emulated library.  Returns (inputs,
    outputs) as lists of byte arrays, the launch info and every buffer."""
    w, B, S, H, D, e = shape
    n = _layout(lib, shape).tensor_bytes // w
    xin = [Buf(n, in_mis[k] if in_mis else 0) for k in range(w)]
    for k, b in enumerate(xin):
        b.view[:] = rand_bytes(n, seed * 1000 + k)
    xout = [Buf(n, out_mis[k] if out_mis else 0) for k in range(w)]
    for b in xout:
        b.view[:] = FILL
    used = [first <= k < first + count for k in range(w)]
    in_ptrs = [b.ptr if (used[k] or not senders_only) else None for k, b in enumerate(xin)]
    h = ctypes.c_void_p()
    assert lib.ua2a_plan(ctypes.byref(h), w, B, S, H, D, e, blocks, None, 0, 0) == 0
    try:
        info = ua.ua2a_launch_info_t()
        assert lib.ua2a_describe_ranks(h, mode, _tab(in_ptrs), _tab([b.ptr for b in xout]),
                                       first, count, ctypes.byref(info)) == 0
        lib.ua2a_emu_reset_counts()
        rc = lib.ua2a_exchange_ranks(h, mode, _tab(in_ptrs), _tab([b.ptr for b in xout]),
                                     first, count, None)
        assert rc == 0, (rc, lib.ua2a_plan_last_error(h))
        # one launch: the per-rank direct kernel (3) or the per-rank LDS kernel (6)
        want_kernel = 6 if info.path == ua.UA2A_PATH_LDS else 3
        assert lib.ua2a_emu_launches() == 1 and lib.ua2a_emu_kernel_count(want_kernel) == 1
    finally:
        lib.ua2a_destroy(h)
    return ([b.view.copy() for b in xin], [b.view.copy() for b in xout], info, xin + xout)


def oracle_ranks(inputs, shape, mode, first, count):
    """The oracle's per-rank exchange on the same bytes, outputs starting at FILL."""
    w, B, S, H, D, e = shape
    ishape = (B, S, H, D) if mode == 0 else (B, S * w, H // w, D)
    oshape = (B, S * w, H // w, D) if mode == 0 else (B, S, H, D)
    xs = [inputs[k].view(DT[e]).reshape(ishape) if first <= k < first + count else None
          for k in range(w)]
    outs = [np.full(int(np.prod(oshape)) * e, FILL, np.uint8).view(DT[e]).reshape(oshape)
            for _ in range(w)]
    oracle.exchange_ranks(xs, outs, mode, first, count)
    return [o.view(np.uint8).ravel() for o in outs]


def sender_ranges(w):
    ranges = [(0, w)] + [(j, 1) for j in range(w)]
    if w > 2:
        ranges.append((1, w - 2))
    return ranges


RANK_SHAPES = [s for s in SHAPES if s[0] <= 8]


@pytest.mark.parametrize("shape", RANK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_emulated_ranks_match_oracle(emu, shape):
    for mode in (0, 1):
        for first, count in sender_ranges(shape[0]):
            xs, ys, info, bufs = emu_ranks(emu, shape, mode, first, count, seed=mode,
                                           senders_only=(count == 1))
            want = oracle_ranks(xs, shape, mode, first, count)
            for k in range(shape[0]):
                assert np.array_equal(ys[k], want[k]), (mode, first, count, k)
            assert all(b.guards_intact() for b in bufs), (mode, first, count)
            assert all(b.view.tobytes() == x.tobytes() for b, x in zip(bufs, xs))   # inputs untouched


@pytest.mark.parametrize("shape", [(4, 1, 40, 8, 128, 2), (3, 1, 5, 3, 7, 2), (2, 2, 9, 4, 64, 2),
                                   (3, 2, 5, 6, 4, 4)], ids=lambda s: "x".join(map(str, s)))
def test_emulated_ranks_misaligned_bases(emu, shape):
    """Every rank's buffers at its own offset from a 64-byte boundary: the
    vector width drops to the alignment they share, the bytes do not change."""
    w, e = shape[0], shape[5]
    for mode in (0, 1):
        in_mis = [(2 * k + 2) * e % 16 for k in range(w)]
        out_mis = [(4 * k) * e % 16 for k in range(w)]
        xs, ys, info, bufs = emu_ranks(emu, shape, mode, 0, w, in_mis, out_mis, seed=3)
        want = oracle_ranks(xs, shape, mode, 0, w)
        assert all(np.array_equal(ys[k], want[k]) for k in range(w)), mode
        assert all(b.guards_intact() for b in bufs)
        assert info.vector_bytes <= 2 * e


@pytest.mark.parametrize("blocks", [1, 3, 7, 64, 100000])
def test_emulated_ranks_grid_cap_does_not_change_bytes(emu, blocks):
    shape = (4, 2, 13, 8, 256, 2)
    for mode in (0, 1):
        for first, count in ((0, 4), (2, 1)):
            xs, ys, info, _ = emu_ranks(emu, shape, mode, first, count, seed=5, blocks=blocks)
            want = oracle_ranks(xs, shape, mode, first, count)
            assert all(np.array_equal(ys[k], want[k]) for k in range(4)), (mode, first, count)
            assert info.grid <= max(blocks, 1) or blocks == 100000


def test_emulated_ranks_slab_grid_beyond_the_hardware_extent(emu):
    """w * B > 65535 slabs along z (mode 0) and B > 65535 along y (mode 1):
    the grid is capped at 65535 and the kernel's loops take the rest."""
    shape = (2, 40000, 1, 2, 1, 1)
    for mode in (0, 1):
        xs, ys, info, _ = emu_ranks(emu, shape, mode, 0, 2, seed=6)
        want = oracle_ranks(xs, shape, mode, 0, 2)
        assert all(np.array_equal(ys[k], want[k]) for k in range(2)), mode
    xs, ys, info, _ = emu_ranks(emu, (2, 70000, 1, 2, 1, 1), 1, 1, 1, seed=7)
    want = oracle_ranks(xs, (2, 70000, 1, 2, 1, 1), 1, 1, 1)
    assert all(np.array_equal(ys[k], want[k]) for k in range(2))


def test_emulated_ranks_tile_counts(emu):
    """One 1 KiB tile per workgroup by default: mode 0 has w*B*count slabs of
    S_local runs, mode 1 w*B slabs of S_local*count runs."""
    w, B, S, H, D, e = shape = (8, 1, 13, 40, 128, 2)        # run 1280 B
    for mode, first, count in ((0, 0, 8), (0, 3, 1), (1, 0, 8), (1, 5, 1)):
        _, _, info, _ = emu_ranks(emu, shape, mode, first, count)
        run = H // w * D * e
        slab = S * run if mode == 0 else S * count * run
        slabs = w * B * count if mode == 0 else w * B
        assert info.tiles == slabs * -(-slab // 1024), (mode, first, count)
        assert info.vector_bytes == 16 and info.block == 64 and info.grid_dims == 3
        assert info.grid == info.tiles


def test_ranks_argument_errors(emu):
    lib = emu
    w, B, S, H, D, e = 2, 1, 4, 4, 8, 2
    h = ctypes.c_void_p()
    assert lib.ua2a_plan(ctypes.byref(h), w, B, S, H, D, e, 0, None, 0, 0) == 0
    n = S * H * D * e * B
    big = Buf(8 * n)
    ins = [big.ptr, big.ptr + n]
    outs = [big.ptr + 2 * n, big.ptr + 3 * n]
    x = lambda i, o, f=0, c=2, mode=0: lib.ua2a_exchange_ranks(
        h, mode, None if i is None else _tab(i), None if o is None else _tab(o), f, c, None)
    try:
        assert x(ins, outs) == ua.UA2A_OK
        assert x(ins, outs, mode=2) == ua.UA2A_ERR_INVALID_ARG
        assert x(None, outs) == ua.UA2A_ERR_INVALID_ARG
        assert x(ins, None) == ua.UA2A_ERR_INVALID_ARG
        assert x(ins, outs, 1, 2) == ua.UA2A_ERR_INVALID_ARG        # past w
        assert x(ins, outs, -1, 1) == ua.UA2A_ERR_INVALID_ARG
        assert x(ins, outs, 0, 0) == ua.UA2A_ERR_INVALID_ARG
        assert x([ins[0], None], outs) == ua.UA2A_ERR_INVALID_ARG   # a sender without input
        assert x([ins[0], None], outs, 0, 1) == ua.UA2A_OK           # non-sender may be NULL
        assert x(ins, [outs[0], None]) == ua.UA2A_ERR_INVALID_ARG   # every output is written
        assert x([ins[0] + 1, ins[1]], outs) == ua.UA2A_ERR_ALIGN
        assert x(ins, [outs[0], outs[1] + 1]) == ua.UA2A_ERR_ALIGN
        assert x(ins, [outs[0], outs[0] + 2]) == ua.UA2A_ERR_ALIAS   # outputs overlap
        assert x(ins, [outs[0], ins[1] + 2]) == ua.UA2A_ERR_ALIAS    # output overlaps a sender
        assert x(ins, [outs[0], ins[1]], 0, 1) == ua.UA2A_OK         # ... a non-sender's is not read
        assert x(ins, [outs[0], outs[0] + n]) == ua.UA2A_OK          # adjacent is fine
        lib.ua2a_emu_set_device(1)
        assert x(ins, outs) == ua.UA2A_ERR_DEVICE
        lib.ua2a_emu_set_device(0)
        lib.ua2a_emu_fail_next_launch(98)
        assert x(ins, outs) == ua.UA2A_ERR_HIP
        assert b"per-rank" in lib.ua2a_plan_last_error(h)
        assert x(ins, outs) == ua.UA2A_ERR_DISABLED
    finally:
        lib.ua2a_emu_set_device(0)
        lib.ua2a_destroy(h)
    # more ranks than the table holds
    assert lib.ua2a_plan(ctypes.byref(h), 65, 1, 1, 65, 1, 1, 0, None, 0, 0) == 0
    try:
        tab = _tab([big.ptr + k for k in range(65)])
        assert lib.ua2a_exchange_ranks(h, 0, tab, tab, 0, 65, None) == ua.UA2A_ERR_SHAPE
    finally:
        lib.ua2a_destroy(h)


def test_emulated_ranks_at_the_largest_table(emu):
    shape = (64, 1, 3, 64, 2, 2)
    for mode in (0, 1):
        for first, count in ((0, 64), (63, 1), (17, 30)):
            xs, ys, _, bufs = emu_ranks(emu, shape, mode, first, count, seed=9)
            want = oracle_ranks(xs, shape, mode, first, count)
            assert all(np.array_equal(ys[k], want[k]) for k in range(64)), (mode, first, count)
            assert all(b.guards_intact() for b in bufs)


# ----------------------------------------------------------- sanitizer build

ASAN_RANKS_DRIVER = r"""
import ctypes, sys
import numpy as np
sys.path.insert(0, {root!r})
import oracle, ulysses_all_re_amd as ua
lib = ua.declare_signatures(ctypes.CDLL({lib!r}))
DT = {{1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}}
for (w, B, S, H, D, e, mode, first, count, mis) in {cases!r}:
    lay = ua.ua2a_layout_t()
    assert lib.ua2a_layout(w, B, S, H, D, e, ctypes.byref(lay)) == 0
    n = lay.tensor_bytes // w
    # exact-size heap blocks per rank (plus the misalignment)
    xin = [(ctypes.c_uint8 * (n + mis))() for _ in range(w)]
    xout = [(ctypes.c_uint8 * (n + mis))() for _ in range(w)]
    for k in range(w):
        np.frombuffer(xin[k], dtype=np.uint8)[mis:] = np.random.default_rng(k).integers(0, 256, n, dtype=np.uint8)
    ip = [ctypes.addressof(b) + mis if first <= k < first + count else None for k, b in enumerate(xin)]
    op = [ctypes.addressof(b) + mis for b in xout]
    h = ctypes.c_void_p()
    assert lib.ua2a_plan(ctypes.byref(h), w, B, S, H, D, e, 0, None, 0, 0) == 0
    tab = lambda p: (ctypes.c_void_p * w)(*p)
    rc = lib.ua2a_exchange_ranks(h, mode, tab(ip), tab(op), first, count, None)
    assert rc == 0, rc
    lib.ua2a_destroy(h)
    ishape = (B, S, H, D) if mode == 0 else (B, S * w, H // w, D)
    oshape = (B, S * w, H // w, D) if mode == 0 else (B, S, H, D)
    xs = [np.frombuffer(xin[k], dtype=np.uint8)[mis:].view(DT[e]).reshape(ishape)
          if first <= k < first + count else None for k in range(w)]
    outs = [np.zeros(oshape, DT[e]) for _ in range(w)]
    oracle.exchange_ranks(xs, outs, mode, first, count)
    for k in range(w):
        got = np.frombuffer(xout[k], dtype=np.uint8)[mis:]
        assert np.array_equal(got, outs[k].view(np.uint8).ravel()), (w, B, S, H, D, e, mode, first, count, mis, k)
    # pack by the sender range into exact-size windows, unpack the same range of receivers
    wins = [(ctypes.c_uint8 * (n + mis))() for _ in range(w)]
    wp = [ctypes.addressof(b) + mis for b in wins]
    h = ctypes.c_void_p()
    assert lib.ua2a_plan(ctypes.byref(h), w, B, S, H, D, e, 0, None, 0, 0) == 0
    assert lib.ua2a_pack_ranks(h, mode, tab(ip), tab(wp), first, count, None) == 0
    assert lib.ua2a_unpack_ranks(h, mode, tab(wp), tab(op), first, count, None) == 0
    lib.ua2a_destroy(h)
    wshape = (B, S * w, H // w, D)
    want_w = [np.zeros(wshape, DT[e]) for _ in range(w)]
    oracle.pack_ranks(xs, want_w, mode, first, count)
    for q in range(w):
        got = np.frombuffer(wins[q], dtype=np.uint8)[mis:]
        assert np.array_equal(got, want_w[q].view(np.uint8).ravel()), ("pack", w, mode, first, count, mis, q)
    want_o = [np.zeros(oshape, DT[e]) for _ in range(w)]
    oracle.unpack_ranks(want_w, want_o, mode, first, count)
    for q in range(first, first + count):
        got = np.frombuffer(xout[q], dtype=np.uint8)[mis:]
        assert np.array_equal(got, want_o[q].view(np.uint8).ravel()), ("unpack", w, mode, first, count, mis, q)
print("asan-ok")
"""


@pytest.mark.slow
def test_emulated_ranks_under_asan(tmp_path):
    lib = emu_build.build(sanitize=True)
    cases = []
    for shape in RANK_SHAPES:
        for mode in (0, 1):
            for first, count in ((0, shape[0]), (shape[0] - 1, 1)):
                cases.append((*shape, mode, first, count, 0))
    for shape in [(3, 1, 5, 3, 7, 2), (4, 1, 40, 8, 128, 2)]:
        for mode in (0, 1):
            cases.append((*shape, mode, 0, shape[0], 2))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = tmp_path / "asan_ranks_driver.py"
    script.write_text(ASAN_RANKS_DRIVER.format(root=root, lib=lib, cases=cases))
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
def ranks_cases(draw):
    w = draw(st.integers(1, 9))
    hl = draw(st.integers(1, 4))
    e = draw(st.sampled_from([1, 2, 4, 8]))
    B = draw(st.integers(1, 3))
    S = draw(st.integers(1, 30))
    D = draw(st.integers(1, 40))
    mode = draw(st.integers(0, 1))
    first = draw(st.integers(0, w - 1))
    count = draw(st.integers(1, w - first))
    in_mis = [draw(st.integers(0, 15)) // e * e for _ in range(w)]
    out_mis = [draw(st.integers(0, 15)) // e * e for _ in range(w)]
    blocks = draw(st.sampled_from([0, 1, 5, 1000]))
    return (w, B, S, w * hl, D, e), mode, first, count, in_mis, out_mis, blocks


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(case=ranks_cases())
def test_emulated_ranks_random_cases_match_oracle(emu, case):
    shape, mode, first, count, in_mis, out_mis, blocks = case
    xs, ys, info, bufs = emu_ranks(emu, shape, mode, first, count, in_mis, out_mis,
                                   seed=sum(shape), blocks=blocks, senders_only=True)
    want = oracle_ranks(xs, shape, mode, first, count)
    assert all(np.array_equal(ys[k], want[k]) for k in range(shape[0])), (case, info.vector_bytes)
    assert all(b.guards_intact() for b in bufs), case


def test_per_rank_path_choice(emu):
    """Short runs take the LDS kernel in mode 0 (any senders) and in mode 1
    when every rank sends; a partial mode-1 sender range and whole-line runs
    take the direct kernel; a forced path is honoured where it applies."""
    lib = emu
    # 64 B runs with w = 8 (a mode-1 tile would read 128 B per head block) and 1 KiB runs
    short, long_ = (8, 1, 40, 8, 32, 2), (4, 1, 40, 8, 256, 2)

    def path(shape, mode, first, count, force=ua.UA2A_PATH_AUTO):
        w, B, S, H, D, e = shape
        n = _layout(lib, shape).tensor_bytes // w
        big = Buf(2 * w * n)
        ins = [big.ptr + k * n for k in range(w)]
        outs = [big.ptr + (w + k) * n for k in range(w)]
        h = ctypes.c_void_p()
        assert lib.ua2a_plan(ctypes.byref(h), w, B, S, H, D, e, 0, None, 0, 0) == 0
        try:
            assert lib.ua2a_plan_set_path(h, force) == 0
            info = ua.ua2a_launch_info_t()
            assert lib.ua2a_describe_ranks(h, mode, _tab(ins), _tab(outs), first, count,
                                           ctypes.byref(info)) == 0
            return info.path, info.lds_rows
        finally:
            lib.ua2a_destroy(h)

    L, Dp = ua.UA2A_PATH_LDS, ua.UA2A_PATH_DIRECT
    assert path(short, 0, 0, 8)[0] == L and path(short, 0, 2, 1)[0] == L
    assert path(short, 1, 0, 8)[0] == L and path(short, 1, 1, 2)[0] == Dp
    assert path(long_, 0, 0, 4)[0] == Dp and path(long_, 1, 0, 4)[0] == Dp
    assert path(long_, 0, 0, 4, L)[0] == L and path(long_, 1, 1, 2, L)[0] == Dp
    assert path(short, 0, 0, 8, Dp) == (Dp, 0)
    assert path(short, 0, 1, 3)[1] > 0
    for shape in (short, long_):
        w = shape[0]
        for mode, first, count in ((0, 0, w), (0, 1, 2), (1, 0, w)):
            for force in (ua.UA2A_PATH_AUTO, L, Dp):
                xs, ys, info, bufs = _forced(lib, shape, mode, first, count, force)
                want = oracle_ranks(xs, shape, mode, first, count)
                assert all(np.array_equal(ys[k], want[k]) for k in range(w)), (shape, mode, force)
                assert all(b.guards_intact() for b in bufs)


def _forced(lib, shape, mode, first, count, force):
    """emu_ranks with a forced path (set on the plan before the call)."""
    w, B, S, H, D, e = shape
    n = _layout(lib, shape).tensor_bytes // w
    xin = [Buf(n) for _ in range(w)]
    for k, b in enumerate(xin):
        b.view[:] = rand_bytes(n, 50 + k)
    xout = [Buf(n) for _ in range(w)]
    for b in xout:
        b.view[:] = FILL
    h = ctypes.c_void_p()
    assert lib.ua2a_plan(ctypes.byref(h), w, B, S, H, D, e, 0, None, 0, 0) == 0
    try:
        assert lib.ua2a_plan_set_path(h, force) == 0
        info = ua.ua2a_launch_info_t()
        tin, tout = _tab([b.ptr for b in xin]), _tab([b.ptr for b in xout])
        assert lib.ua2a_describe_ranks(h, mode, tin, tout, first, count, ctypes.byref(info)) == 0
        assert lib.ua2a_exchange_ranks(h, mode, tin, tout, first, count, None) == 0
    finally:
        lib.ua2a_destroy(h)
    return [b.view.copy() for b in xin], [b.view.copy() for b in xout], info, xin + xout


# -------------------------------------------------- pack and unpack (windows)

def emu_pack_unpack(lib, shape, mode, first, count, mis=None, seed=0, path=ua.UA2A_PATH_AUTO, blocks=0):
    """Pack senders [first, first+count) into every window, then unpack
    receivers [first, first+count) (the same range, reused as receivers).
    Returns (inputs, windows after pack, outputs after unpack) as byte arrays,
    the launch counts, and every buffer."""
    w, B, S, H, D, e = shape
    n = _layout(lib, shape).tensor_bytes // w
    m = mis or [0] * w
    xin = [Buf(n, m[k]) for k in range(w)]
    for k, b in enumerate(xin):
        b.view[:] = rand_bytes(n, seed * 1000 + k)
    wins = [Buf(n, m[(k + 1) % w]) for k in range(w)]
    for b in wins:
        b.view[:] = FILL
    outs = [Buf(n, m[(k + 2) % w]) for k in range(w)]
    for b in outs:
        b.view[:] = FILL
    used = [first <= k < first + count for k in range(w)]
    h = ctypes.c_void_p()
    assert lib.ua2a_plan(ctypes.byref(h), w, B, S, H, D, e, blocks, None, 0, 0) == 0
    try:
        assert lib.ua2a_plan_set_path(h, path) == 0
        lib.ua2a_emu_reset_counts()
        rc = lib.ua2a_pack_ranks(h, mode, _tab([b.ptr if used[k] else None for k, b in enumerate(xin)]),
                                 _tab([b.ptr for b in wins]), first, count, None)
        assert rc == 0, (rc, lib.ua2a_plan_last_error(h))
        packed = [b.view.copy() for b in wins]
        launches_pack = lib.ua2a_emu_launches()
        pack_kernel = lib.ua2a_emu_kernel_count(8)
        lib.ua2a_emu_reset_counts()
        rc = lib.ua2a_unpack_ranks(h, mode, _tab([b.ptr if used[k] else None for k, b in enumerate(wins)]),
                                   _tab([b.ptr if used[k] else None for k, b in enumerate(outs)]),
                                   first, count, None)
        assert rc == 0, (rc, lib.ua2a_plan_last_error(h))
        launches_unpack = lib.ua2a_emu_launches()
    finally:
        lib.ua2a_destroy(h)
    return ([b.view.copy() for b in xin], packed, [b.view.copy() for b in outs],
            (launches_pack, pack_kernel, launches_unpack), xin + wins + outs)


def oracle_pack_unpack(inputs, shape, mode, first, count):
    w, B, S, H, D, e = shape
    dt = DT[e]
    ishape = (B, S, H, D) if mode == 0 else (B, S * w, H // w, D)
    wshape = (B, S * w, H // w, D)
    oshape = wshape if mode == 0 else (B, S, H, D)
    xs = [x.view(dt).reshape(ishape) for x in inputs]
    wins = [np.full(wshape, FILL, np.uint8).view(dt) if e == 1 else
            np.frombuffer(bytes([FILL]) * (int(np.prod(wshape)) * e), dtype=dt).reshape(wshape).copy()
            for _ in range(w)]
    oracle.pack_ranks([xs[k] if first <= k < first + count else None for k in range(w)], wins, mode,
                      first, count)
    outs = [np.frombuffer(bytes([FILL]) * (int(np.prod(oshape)) * e), dtype=dt).reshape(oshape).copy()
            for _ in range(w)]
    oracle.unpack_ranks(wins, outs, mode, first, count)
    return ([wn.view(np.uint8).ravel() for wn in wins], [o.view(np.uint8).ravel() for o in outs])


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_emulated_pack_unpack_match_oracle(emu, shape):
    """Pack of every sender range and unpack of the same range of receivers,
    both modes, against the oracle's pack and unpack; windows and outputs
    outside the ranges keep their fill; guards intact."""
    w = shape[0]
    ranges = [(0, w)] + [(k, 1) for k in range(w)] + ([(1, w - 1)] if w > 2 else [])
    for mode in (0, 1):
        for first, count in ranges:
            x, packed, outs, (lp, pk, lu), bufs = emu_pack_unpack(emu, shape, mode, first, count, seed=mode + 5)
            want_w, want_o = oracle_pack_unpack(x, shape, mode, first, count)
            for q in range(w):
                assert np.array_equal(packed[q], want_w[q]), (mode, first, count, q)
                assert np.array_equal(outs[q], want_o[q]), (mode, first, count, q)
            assert lp == 1 and lu == count
            assert pk == (1 if mode == 1 else 0)      # mode 0 packs with the per-rank exchange
            assert all(b.guards_intact() for b in bufs)


@pytest.mark.parametrize("path", [ua.UA2A_PATH_AUTO, ua.UA2A_PATH_DIRECT, ua.UA2A_PATH_LDS],
                         ids=["auto", "direct", "lds"])
@pytest.mark.parametrize("shape", [(3, 2, 5, 3, 7, 2), (4, 1, 40, 8, 128, 2), (2, 2, 9, 4, 64, 2),
                                   (5, 3, 37, 10, 3, 1), (3, 2, 11, 6, 5, 8)],
                         ids=lambda s: "x".join(map(str, s)))
def test_emulated_pack_then_unpack_is_the_exchange(emu, shape, path):
    """One pack per sender and one unpack of every receiver equal the
    oracle's exchange, with misaligned bases too (narrower vectors)."""
    w, B, S, H, D, e = shape
    for mis in (None, [e * ((k % 3) + 1) for k in range(w)]):
        for mode in (0, 1):
            x, _, outs, _, bufs = emu_pack_unpack(emu, shape, mode, 0, w, mis=mis, seed=mode + 9, path=path)
            xs = np.stack([a.view(DT[e]) for a in x]).reshape(
                (w, B, S, H, D) if mode == 0 else (w, B, S * w, H // w, D))
            want = oracle.exchange(xs, mode, w)
            assert np.array_equal(np.stack(outs).view(DT[e]).reshape(want.shape), want), (mode, mis)
            assert all(b.guards_intact() for b in bufs)


@pytest.mark.parametrize("blocks", [1, 5, 1000])
def test_emulated_pack_with_a_capped_grid(emu, blocks):
    shape = (4, 3, 50, 8, 16, 2)
    for mode in (0, 1):
        x, packed, outs, _, _ = emu_pack_unpack(emu, shape, mode, 0, 4, seed=3, blocks=blocks)
        want_w, want_o = oracle_pack_unpack(x, shape, mode, 0, 4)
        assert all(np.array_equal(a, b) for a, b in zip(packed, want_w)), mode
        assert all(np.array_equal(a, b) for a, b in zip(outs, want_o)), mode


def test_emulated_pack_unpack_argument_errors(emu):
    w, B, S, H, D, e = 2, 1, 4, 2, 8, 2
    n = _layout(emu, (w, B, S, H, D, e)).tensor_bytes // w
    bufs = [Buf(n) for _ in range(6)]
    xs, wins, outs = [b.ptr for b in bufs[:2]], [b.ptr for b in bufs[2:4]], [b.ptr for b in bufs[4:]]
    h = ctypes.c_void_p()
    assert emu.ua2a_plan(ctypes.byref(h), w, B, S, H, D, e, 0, None, 0, 0) == 0
    assert emu.ua2a_pack_ranks(h, 2, _tab(xs), _tab(wins), 0, 2, None) == ua.UA2A_ERR_INVALID_ARG
    assert emu.ua2a_pack_ranks(h, 1, _tab(xs), _tab([wins[0], None]), 0, 1, None) == ua.UA2A_ERR_INVALID_ARG
    assert emu.ua2a_pack_ranks(h, 1, _tab(xs), _tab([wins[0], wins[0]]), 0, 2, None) == ua.UA2A_ERR_ALIAS
    assert emu.ua2a_pack_ranks(h, 1, _tab(xs), _tab([xs[1], wins[1]]), 0, 2, None) == ua.UA2A_ERR_ALIAS
    assert emu.ua2a_pack_ranks(h, 1, _tab(xs), _tab([wins[0] + 1, wins[1]]), 0, 2, None) == ua.UA2A_ERR_ALIGN
    assert emu.ua2a_unpack_ranks(h, 1, _tab(wins), _tab(outs), 1, 2, None) == ua.UA2A_ERR_INVALID_ARG
    assert emu.ua2a_unpack_ranks(h, 1, _tab(wins), _tab([wins[1], outs[1]]), 0, 2, None) == ua.UA2A_ERR_ALIAS
    assert emu.ua2a_unpack_ranks(h, 1, _tab(wins), _tab([outs[0], outs[0]]), 0, 2, None) == ua.UA2A_ERR_ALIAS
    assert emu.ua2a_unpack_ranks(h, 1, _tab([None, wins[1]]), _tab([None, outs[1]]), 1, 1, None) == 0
    emu.ua2a_emu_set_device(1)
    assert emu.ua2a_pack_ranks(h, 1, _tab(xs), _tab(wins), 0, 2, None) == ua.UA2A_ERR_DEVICE
    assert emu.ua2a_unpack_ranks(h, 1, _tab(wins), _tab(outs), 0, 2, None) == ua.UA2A_ERR_DEVICE
    emu.ua2a_emu_set_device(0)
    assert emu.ua2a_plan_last_error(h) == b""
    emu.ua2a_destroy(h)
