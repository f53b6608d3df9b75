"""CPU oracle of the Ulysses all_to_all_4D head/sequence exchange.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are its only callers.  The product path
(``ulysses_all_re_amd``) never imports it, and it imports nothing from there.

The arithmetic lives in ``ua2a_oracle.c`` as plain nested loops (see the
header of that file for the page and method each loop follows); this module
only builds that file with gcc, loads it with ctypes and marshals numpy
arrays.

Shapes follow the FastVideo ``ulysses_a2a`` page (method ``run_armed``): the
w rank tensors are stacked rank-major in one array,
    mode 0 input  [w, B, S_local, H, D]      -> output [w, B, S_local*w, H//w, D]
    mode 1 input  [w, B, S_global, H_local, D] -> output [w, B, S_global//w, H_local*w, D]
and elements are moved as raw bit patterns (any numpy dtype of 1, 2, 4 or 8
bytes; bf16 travels as uint16/int16).

``exchange_ranks`` runs the exchange between separate per-rank arrays,
restricted to a range of sending ranks; ``pack_ranks`` and ``unpack_ranks``
run it in two steps through one receive window per receiving rank (see
``ua2a_oracle.c``).

``source_indices`` gives, for chosen output positions, the input position
each one comes from (the same definitions, one element at a time), for
checking outputs too large to copy whole to the host.

Parity pins (tests/test_oracle_pins.py): closed-form shapes, w = 1 identity,
mode1(mode0(x)) == x and mode0(mode1(y)) == y, chunked == unchunked,
agreement with an all-to-all over torch.distributed's gloo backend in w
processes, agreement with numpy reshape/transpose, hand-derived worked
examples under tests/golden/, bijection of the element multiset; for the
per-rank form, the numpy permutation masked by the source rank of every
element, and the union of single-sender calls; for pack and unpack, numpy
slices and transposes of each window, and pack followed by unpack equal to
the numpy exchange.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "ua2a_oracle.c")
LIBRARY = os.path.join(_HERE, "libua2a_oracle.so")

_lib = None


def build() -> str:
    """Compile the oracle with gcc into oracle/libua2a_oracle.so."""
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-Werror",
           "-shared", "-fPIC", SOURCE, "-o", LIBRARY + ".tmp"]
    subprocess.check_call(cmd)
    os.replace(LIBRARY + ".tmp", LIBRARY)
    return LIBRARY


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        build()
    lib = ctypes.CDLL(LIBRARY)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    for name in ("ua2a_oracle_mode0", "ua2a_oracle_mode1"):
        fn = getattr(lib, name)
        fn.argtypes = [i32, i64, i64, i64, i64, i32, vp, vp]
        fn.restype = ctypes.c_int
    lib.ua2a_oracle_chunked.argtypes = [i32, i32, i64, i64, i64, i64, i32, vp, vp]
    lib.ua2a_oracle_chunked.restype = ctypes.c_int
    for name in ("ua2a_oracle_ranks", "ua2a_oracle_pack_ranks", "ua2a_oracle_unpack_ranks"):
        fn = getattr(lib, name)
        fn.argtypes = [i32, i32, i64, i64, i64, i64, i32, vp, vp, i32, i32]
        fn.restype = ctypes.c_int
    lib.ua2a_oracle_source_index.argtypes = [i32, i32, i64, i64, i64, i64, i64]
    lib.ua2a_oracle_source_index.restype = i64
    lib.ua2a_oracle_source_indices.argtypes = [i32, i32, i64, i64, i64, i64, vp, i64, vp]
    lib.ua2a_oracle_source_indices.restype = ctypes.c_int
    _lib = lib
    return lib


class OracleError(ValueError):
    """Raised when the oracle rejects its arguments (code from ua2a_oracle.c)."""

    def __init__(self, code: int):
        super().__init__(f"oracle rejected the call (code {code})")
        self.code = code


def local_shape(x_shape, mode: int, w: int):
    """(B, S_local, H, D) of a rank-stacked input, derived the way run_armed does."""
    if len(x_shape) != 5 or x_shape[0] != w:
        raise ValueError(f"expected a rank-stacked [w={w}, B, S, H, D] array, got {tuple(x_shape)}")
    _, B, S, Hx, D = x_shape
    if mode == 0:
        return B, S, Hx, D
    if mode == 1:
        if S % w:
            raise ValueError("mode 1 needs S_global divisible by w")
        return B, S // w, Hx * w, D
    raise ValueError("mode must be 0 or 1")


def exchange(x: np.ndarray, mode: int, w: int, chunked: bool = False) -> np.ndarray:
    """Run the oracle on a rank-stacked array and return a fresh output array."""
    x = np.ascontiguousarray(x)
    B, S_local, H, D = local_shape(x.shape, mode, w)
    if H % w:
        raise OracleError(-2)
    if mode == 0:
        out = np.empty((w, B, S_local * w, H // w, D), dtype=x.dtype)
    else:
        out = np.empty((w, B, S_local, H, D), dtype=x.dtype)
    lib = _load()
    e = x.dtype.itemsize
    ip, op = x.ctypes.data, out.ctypes.data
    if chunked:
        rc = lib.ua2a_oracle_chunked(mode, w, B, S_local, H, D, e, ip, op)
    elif mode == 0:
        rc = lib.ua2a_oracle_mode0(w, B, S_local, H, D, e, ip, op)
    else:
        rc = lib.ua2a_oracle_mode1(w, B, S_local, H, D, e, ip, op)
    if rc != 0:
        raise OracleError(rc)
    return out


def exchange_ranks(xs, outs, mode: int, first: int = 0, count=None) -> None:
    """The exchange between separate per-rank arrays, in place into `outs`.

    xs[k] is rank k's input without the leading rank axis (mode 0:
    [B, S_local, H, D]; mode 1: [B, S_global, H_local, D]); only the entries of
    the sending ranks [first, first + count) are read and the others may be
    None.  outs[k] is rank k's output, fully given: only elements whose source
    rank is a sender are written.
    """
    w = len(outs)
    count = w - first if count is None else count
    if len(xs) != w:
        raise ValueError("xs and outs must both hold one entry per rank")
    senders = [xs[k] for k in range(first, first + count)]
    if not senders or any(x is None for x in senders):
        raise OracleError(-1)
    ref = senders[0]
    if any(x.shape != ref.shape or x.dtype != ref.dtype or not x.flags.c_contiguous for x in senders):
        raise ValueError("sender inputs must share one shape and dtype and be C-contiguous")
    B, S_local, H, D = local_shape((w, *ref.shape), mode, w)
    if H % w:
        raise OracleError(-2)
    out_shape = (B, S_local * w, H // w, D) if mode == 0 else (B, S_local, H, D)
    for o in outs:
        if o.shape != out_shape or o.dtype != ref.dtype or not o.flags.c_contiguous:
            raise ValueError(f"every output must be a C-contiguous {out_shape} {ref.dtype} array")
    vp = ctypes.c_void_p
    in_tab = (vp * w)(*[None if x is None else x.ctypes.data for x in xs])
    out_tab = (vp * w)(*[o.ctypes.data for o in outs])
    rc = _load().ua2a_oracle_ranks(mode, w, B, S_local, H, D, ref.dtype.itemsize,
                                   ctypes.cast(in_tab, vp), ctypes.cast(out_tab, vp), first, count)
    if rc != 0:
        raise OracleError(rc)


def _window_shape(B, S_local, H, D, w):
    return (B, S_local * w, H // w, D)


def pack_ranks(xs, wins, mode: int, first: int = 0, count=None) -> None:
    """Pack, in place into `wins`: wins[q] is receiver q's window
    [B, S_local*w, H//w, D]; token block k of each plane receives what sender
    k (in [first, first + count)) sends q.  xs as for exchange_ranks."""
    w = len(wins)
    count = w - first if count is None else count
    if len(xs) != w:
        raise ValueError("xs and wins must both hold one entry per rank")
    senders = [xs[k] for k in range(first, first + count)]
    if not senders or any(x is None for x in senders):
        raise OracleError(-1)
    ref = senders[0]
    if any(x.shape != ref.shape or x.dtype != ref.dtype or not x.flags.c_contiguous for x in senders):
        raise ValueError("sender inputs must share one shape and dtype and be C-contiguous")
    B, S_local, H, D = local_shape((w, *ref.shape), mode, w)
    if H % w:
        raise OracleError(-2)
    for wn in wins:
        if wn.shape != _window_shape(B, S_local, H, D, w) or wn.dtype != ref.dtype or not wn.flags.c_contiguous:
            raise ValueError("every window must be a C-contiguous [B, S_local*w, H//w, D] array")
    vp = ctypes.c_void_p
    in_tab = (vp * w)(*[None if x is None else x.ctypes.data for x in xs])
    win_tab = (vp * w)(*[x.ctypes.data for x in wins])
    rc = _load().ua2a_oracle_pack_ranks(mode, w, B, S_local, H, D, ref.dtype.itemsize,
                                        ctypes.cast(in_tab, vp), ctypes.cast(win_tab, vp), first, count)
    if rc != 0:
        raise OracleError(rc)


def unpack_ranks(wins, outs, mode: int, first: int = 0, count=None) -> None:
    """Unpack receivers [first, first + count), in place into `outs`: outs[q]
    (mode 0: [B, S_local*w, H//w, D]; mode 1: [B, S_local, H, D]) from window
    wins[q]; other entries are not touched (and may be None)."""
    w = len(wins)
    count = w - first if count is None else count
    if len(outs) != w:
        raise ValueError("wins and outs must both hold one entry per rank")
    used = [(wins[q], outs[q]) for q in range(first, first + count)]
    if not used or any(a is None or b is None for a, b in used):
        raise OracleError(-1)
    ref = used[0][0]
    B, S_g, Hl, D = ref.shape
    if S_g % w:
        raise ValueError("a window holds w token blocks")
    S_local, H = S_g // w, Hl * w
    out_shape = _window_shape(B, S_local, H, D, w) if mode == 0 else (B, S_local, H, D)
    for a, b in used:
        if a.shape != ref.shape or a.dtype != ref.dtype or not a.flags.c_contiguous:
            raise ValueError("windows must share one shape and dtype and be C-contiguous")
        if b.shape != out_shape or b.dtype != ref.dtype or not b.flags.c_contiguous:
            raise ValueError(f"every used output must be a C-contiguous {out_shape} array")
    vp = ctypes.c_void_p
    win_tab = (vp * w)(*[None if x is None else x.ctypes.data for x in wins])
    out_tab = (vp * w)(*[None if x is None else x.ctypes.data for x in outs])
    rc = _load().ua2a_oracle_unpack_ranks(mode, w, B, S_local, H, D, ref.dtype.itemsize,
                                          ctypes.cast(win_tab, vp), ctypes.cast(out_tab, vp), first, count)
    if rc != 0:
        raise OracleError(rc)


def source_indices(mode: int, w: int, B: int, S_local: int, H: int, D: int,
                   out_index: np.ndarray) -> np.ndarray:
    """Input positions of the elements the exchange writes at `out_index` (int64 array)."""
    idx = np.ascontiguousarray(out_index, dtype=np.int64)
    src = np.empty_like(idx)
    rc = _load().ua2a_oracle_source_indices(mode, w, B, S_local, H, D, idx.ctypes.data,
                                             idx.size, src.ctypes.data)
    if rc != 0:
        raise OracleError(rc)
    return src


def raw_call(fn_name: str, *args) -> int:
    """Call one oracle entry point with raw arguments (for argument-check tests)."""
    return getattr(_load(), fn_name)(*args)
