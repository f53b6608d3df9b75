"""Python binding of the MI355X Ulysses all_to_all_4D exchange library (libua2a.so).

Argument marshalling only: every byte of the exchange is moved by the HIP
kernels in libua2a.so.  PyTorch is used for device memory and streams.

The functions mirror the C ABI of include/ua2a.h one to one
(``ua2a_layout``, ``ua2a_plan``, ``ua2a_exchange``,
``ua2a_exchange_chunked_noalloc``, ``ua2a_exchange_ranks``, ``ua2a_pack_ranks``,
``ua2a_unpack_ranks``,
``ua2a_exchange_publish``, ``ua2a_wait_credits``, ``ua2a_destroy``,
``ua2a_status_string``, ``ua2a_plan_last_error``, ``ua2a_plan_set_path``,
``ua2a_describe``, ``ua2a_describe_ranks``) and raise :class:`UA2AError` on a
non-zero status.
:class:`Plan` wraps them for torch tensors laid out rank-stacked:

    mode 0 input  [w, B, S_local, H, D]        -> output [w, B, S_local*w, H//w, D]
    mode 1 input  [w, B, S_local*w, H//w, D]   -> output [w, B, S_local, H, D]

(FastVideo ``ulysses_a2a`` API page, method ``run_armed``: mode 0 scatters
heads and gathers the sequence, mode 1 is its inverse, chunked runs the same
exchange one batch plane at a time through a window sized for one plane.)
``Plan.exchange_ranks`` runs it between per-rank tensors (one allocation
each, the ranks' shapes without the leading w), optionally only for the runs
a range of ranks sends.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG_DIR, "libua2a.so")

UA2A_OK = 0
UA2A_ERR_INVALID_ARG = -1
UA2A_ERR_SHAPE = -2
UA2A_ERR_ALIGN = -3
UA2A_ERR_ALIAS = -4
UA2A_ERR_CAPACITY = -5
UA2A_ERR_DEVICE = -6
UA2A_ERR_HIP = -7
UA2A_ERR_DISABLED = -8
UA2A_ERR_NOMEM = -9

UA2A_PATH_AUTO = 0
UA2A_PATH_DIRECT = 1
UA2A_PATH_LDS = 2

UA2A_CHUNKED_ONE_LAUNCH = 1

UA2A_NOALLOC_WINDOW_BYTES = 64 * 1024 * 1024   # the library's own window (no-allocation entry point)

# every symbol include/ua2a.h declares
EXPORTED = (
    "ua2a_layout", "ua2a_plan", "ua2a_exchange", "ua2a_exchange_chunked_noalloc",
    "ua2a_exchange_ranks", "ua2a_pack_ranks", "ua2a_unpack_ranks", "ua2a_destroy",
    "ua2a_status_string", "ua2a_plan_last_error", "ua2a_plan_set_path", "ua2a_describe",
    "ua2a_describe_ranks", "ua2a_exchange_publish", "ua2a_wait_credits",
)

MAX_RANK_TABLE = 64     # largest w that ua2a_exchange_ranks accepts


class ua2a_layout_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "H_local", "S_global", "run_bytes", "tensor_elems", "tensor_bytes",
        "window_bytes", "moved_bytes")]


class ua2a_launch_info_t(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("vector_bytes", ctypes.c_int32),
                ("block", ctypes.c_int32), ("launches", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("tiles", ctypes.c_int64),
                ("lds_rows", ctypes.c_int32), ("grid_dims", ctypes.c_int32),
                ("chunked_form", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("lds_planes", ctypes.c_int32)]


class UA2AError(RuntimeError):
    """A non-zero ua2a status."""

    def __init__(self, code: int, what: str, detail: str = ""):
        msg = f"{what}: {ua2a_status_string(code)} ({code})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)
        self.code = code


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libua2a.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise RuntimeError(
            f"{LIBRARY} is missing: build it with `python -m ulysses_all_re_amd.build` "
            "(the exchange has no non-HIP implementation)")
    _lib = declare_signatures(ctypes.CDLL(LIBRARY))
    return _lib


def declare_signatures(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Set ctypes argument/return types of the C ABI on a loaded library."""
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    sig = {
        "ua2a_layout": ([i32, i64, i64, i64, i64, i32, ctypes.POINTER(ua2a_layout_t)], ctypes.c_int),
        "ua2a_plan": ([ctypes.POINTER(vp), i32, i64, i64, i64, i64, i32, i32, vp, i64, i32], ctypes.c_int),
        "ua2a_exchange": ([vp, i32, i32, vp, vp, vp], ctypes.c_int),
        "ua2a_exchange_chunked_noalloc": ([vp, i32, vp, vp, vp], ctypes.c_int),
        "ua2a_destroy": ([vp], ctypes.c_int),
        "ua2a_status_string": ([i32], ctypes.c_char_p),
        "ua2a_plan_last_error": ([vp], ctypes.c_char_p),
        "ua2a_plan_set_path": ([vp, i32], ctypes.c_int),
        "ua2a_describe": ([vp, i32, i32, vp, vp, ctypes.POINTER(ua2a_launch_info_t)], ctypes.c_int),
        "ua2a_exchange_ranks": ([vp, i32, vp, vp, i32, i32, vp], ctypes.c_int),
        "ua2a_pack_ranks": ([vp, i32, vp, vp, i32, i32, vp], ctypes.c_int),
        "ua2a_unpack_ranks": ([vp, i32, vp, vp, i32, i32, vp], ctypes.c_int),
        "ua2a_describe_ranks": ([vp, i32, vp, vp, i32, i32, ctypes.POINTER(ua2a_launch_info_t)],
                                ctypes.c_int),
        "ua2a_exchange_publish": ([vp, i32, vp, vp, vp, i32, vp], ctypes.c_int),
        "ua2a_wait_credits": ([vp, i64, i64, ctypes.c_uint32, ctypes.c_uint32, vp, vp], ctypes.c_int),
    }
    for name, (argtypes, restype) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = restype
    return lib


# ------------------------------------------------------------ C ABI mirror

def ua2a_status_string(status: int) -> str:
    return load_library().ua2a_status_string(status).decode()


def ua2a_layout(w: int, B: int, S_local: int, H: int, D: int, elem_bytes: int) -> dict:
    lay = ua2a_layout_t()
    rc = load_library().ua2a_layout(w, B, S_local, H, D, elem_bytes, ctypes.byref(lay))
    if rc != UA2A_OK:
        raise UA2AError(rc, "ua2a_layout")
    return {name: getattr(lay, name) for name, _ in ua2a_layout_t._fields_}


def ua2a_plan(w: int, B: int, S_local: int, H: int, D: int, elem_bytes: int, blocks: int = 0,
              window: int = 0, window_bytes: int = 0, device: int = 0) -> int:
    """Create a plan; returns the opaque handle (an int)."""
    h = ctypes.c_void_p()
    rc = load_library().ua2a_plan(ctypes.byref(h), w, B, S_local, H, D, elem_bytes, blocks,
                                  window or None, window_bytes, device)
    if rc != UA2A_OK:
        raise UA2AError(rc, "ua2a_plan")
    return h.value


def ua2a_plan_last_error(plan: int) -> str:
    return load_library().ua2a_plan_last_error(plan).decode()


def ua2a_exchange(plan: int, mode: int, chunked: int, inp: int, out: int, stream: int = 0) -> None:
    """Enqueue one exchange on `stream` (raw device pointers and a hipStream_t)."""
    rc = load_library().ua2a_exchange(plan, mode, chunked, inp or None, out or None, stream or None)
    if rc != UA2A_OK:
        raise UA2AError(rc, "ua2a_exchange", ua2a_plan_last_error(plan) if plan else "")


def ua2a_exchange_chunked_noalloc(plan: int, mode: int, inp: int, out: int, stream: int = 0) -> None:
    """Enqueue one chunked exchange through the library's own window (no allocation)."""
    rc = load_library().ua2a_exchange_chunked_noalloc(plan, mode, inp or None, out or None, stream or None)
    if rc != UA2A_OK:
        raise UA2AError(rc, "ua2a_exchange_chunked_noalloc", ua2a_plan_last_error(plan) if plan else "")


def _table(ptrs):
    """A C array of device pointers (None or 0 for an unused entry)."""
    return (ctypes.c_void_p * len(ptrs))(*[p or None for p in ptrs])


def ua2a_exchange_ranks(plan: int, mode: int, in_ptrs, out_ptrs, first: int, count: int,
                        stream: int = 0) -> None:
    """Enqueue the exchange between per-rank allocations (lists of raw device
    pointers, indexed by sending / receiving rank) for senders [first, first+count)."""
    rc = load_library().ua2a_exchange_ranks(plan, mode, _table(in_ptrs) if in_ptrs is not None else None,
                                            _table(out_ptrs) if out_ptrs is not None else None,
                                            first, count, stream or None)
    if rc != UA2A_OK:
        raise UA2AError(rc, "ua2a_exchange_ranks", ua2a_plan_last_error(plan) if plan else "")


def ua2a_pack_ranks(plan: int, mode: int, in_ptrs, win_ptrs, first: int, count: int,
                    stream: int = 0) -> None:
    """Enqueue the pack of senders [first, first+count) into every receiver's window."""
    rc = load_library().ua2a_pack_ranks(plan, mode, _table(in_ptrs) if in_ptrs is not None else None,
                                        _table(win_ptrs) if win_ptrs is not None else None,
                                        first, count, stream or None)
    if rc != UA2A_OK:
        raise UA2AError(rc, "ua2a_pack_ranks", ua2a_plan_last_error(plan) if plan else "")


def ua2a_unpack_ranks(plan: int, mode: int, win_ptrs, out_ptrs, first: int, count: int,
                      stream: int = 0) -> None:
    """Enqueue the unpack of receivers [first, first+count) from their windows."""
    rc = load_library().ua2a_unpack_ranks(plan, mode, _table(win_ptrs) if win_ptrs is not None else None,
                                          _table(out_ptrs) if out_ptrs is not None else None,
                                          first, count, stream or None)
    if rc != UA2A_OK:
        raise UA2AError(rc, "ua2a_unpack_ranks", ua2a_plan_last_error(plan) if plan else "")


def ua2a_describe_ranks(plan: int, mode: int, in_ptrs, out_ptrs, first: int, count: int) -> dict:
    info = ua2a_launch_info_t()
    rc = load_library().ua2a_describe_ranks(plan, mode, _table(in_ptrs) if in_ptrs is not None else None,
                                            _table(out_ptrs) if out_ptrs is not None else None,
                                            first, count, ctypes.byref(info))
    if rc != UA2A_OK:
        raise UA2AError(rc, "ua2a_describe_ranks")
    return {name: getattr(info, name) for name, _ in ua2a_launch_info_t._fields_}


def ua2a_exchange_publish(plan: int, mode: int, inp: int, out: int, credits: int, parts: int,
                          stream: int = 0) -> None:
    rc = load_library().ua2a_exchange_publish(plan, mode, inp or None, out or None, credits or None,
                                              parts, stream or None)
    if rc != UA2A_OK:
        raise UA2AError(rc, "ua2a_exchange_publish", ua2a_plan_last_error(plan) if plan else "")


def ua2a_wait_credits(credits: int, first: int, count: int, target: int, spin_limit: int,
                      status: int, stream: int = 0) -> None:
    rc = load_library().ua2a_wait_credits(credits or None, first, count, target & 0xFFFFFFFF,
                                          spin_limit, status or None, stream or None)
    if rc != UA2A_OK:
        raise UA2AError(rc, "ua2a_wait_credits")


def wait_credits(credits, first: int, count: int, target: int, status, spin_limit: int = 1 << 22,
                 stream=None) -> None:
    """Enqueue a wait on `stream` (default: torch's current stream) until
    credits[first : first+count] (a uint32/int32 device tensor, one counter per
    receiving rank) reach `target`; `status` (an int32 device tensor, zeroed by
    the caller) becomes 1 on a time-out."""
    import torch
    if credits.element_size() != 4 or status.element_size() != 4:
        raise TypeError("credits and status must be 4-byte integer tensors")
    if not (credits.is_contiguous() and credits.is_cuda and status.is_cuda):
        raise ValueError("credits and status must be contiguous device tensors")
    if status.device != credits.device:
        raise ValueError(f"status is on {status.device}, credits are on {credits.device}")
    if first < 0 or count < 1 or first + count > credits.numel():
        raise ValueError(f"slab range [{first}, {first + count}) is outside the {credits.numel()} counters")
    if stream is None:
        stream = torch.cuda.current_stream(credits.device)
    with torch.cuda.device(credits.device):     # launch on the counters' device
        ua2a_wait_credits(credits.data_ptr(), first, count, target, spin_limit, status.data_ptr(),
                          stream.cuda_stream)


def ua2a_destroy(plan: int) -> None:
    load_library().ua2a_destroy(plan)


def ua2a_plan_set_path(plan: int, path: int) -> None:
    rc = load_library().ua2a_plan_set_path(plan, path)
    if rc != UA2A_OK:
        raise UA2AError(rc, "ua2a_plan_set_path")


def ua2a_describe(plan: int, mode: int, chunked: int, inp: int, out: int) -> dict:
    info = ua2a_launch_info_t()
    rc = load_library().ua2a_describe(plan, mode, chunked, inp or None, out or None,
                                      ctypes.byref(info))
    if rc != UA2A_OK:
        raise UA2AError(rc, "ua2a_describe")
    return {name: getattr(info, name) for name, _ in ua2a_launch_info_t._fields_}


# ------------------------------------------------------------- torch wrapper

def _current_raw_stream(device) -> int:
    """torch's current stream on `device` as a raw hipStream_t (0: the null
    stream), without building a Stream object where torch offers that."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(device.index)
    return torch.cuda.current_stream(device).cuda_stream


class Plan:
    """A ua2a plan bound to torch tensors on one device.

    ``window``: optional device tensor used as the one-plane window of
    chunked exchanges (at least ``layout['window_bytes']`` bytes); the plan
    keeps a reference to it for its own lifetime.
    """

    def __init__(self, w: int, B: int, S_local: int, H: int, D: int, dtype, blocks: int = 0,
                 window=None, device=None):
        import torch
        self.w, self.B, self.S_local, self.H, self.D = w, B, S_local, H, D
        self.dtype = dtype
        self.elem_bytes = torch.empty((), dtype=dtype).element_size()
        dev = torch.device("cuda") if device is None else torch.device(device)
        if dev.type != "cuda":
            raise ValueError(f"a plan lives on a GPU, not on {dev}")
        self.device = torch.device("cuda", torch.cuda.current_device() if dev.index is None
                                   else dev.index)
        self.layout = ua2a_layout(w, B, S_local, H, D, self.elem_bytes)
        self.window = window
        wptr, wbytes = 0, 0
        if window is not None:
            if window.device != self.device:
                raise ValueError(f"window is on {window.device}, plan is on {self.device}")
            wptr, wbytes = window.data_ptr(), window.numel() * window.element_size()
        self.handle = ua2a_plan(w, B, S_local, H, D, self.elem_bytes, blocks, wptr, wbytes,
                                self.device.index)

    @staticmethod
    def window_bytes(w: int, B: int, S_local: int, H: int, D: int, elem_bytes: int) -> int:
        """Bytes a chunked exchange of this shape needs in its window (one plane of every rank)."""
        return ua2a_layout(w, B, S_local, H, D, elem_bytes)["window_bytes"]

    def in_shape(self, mode: int):
        w, B, S, H, D = self.w, self.B, self.S_local, self.H, self.D
        return (w, B, S, H, D) if mode == 0 else (w, B, S * w, H // w, D)

    def out_shape(self, mode: int):
        return self.in_shape(1 - mode)

    def _on_device(self, fn, *args):
        """Call fn(*args) with the plan's device current (the library checks it)."""
        import torch
        if torch.cuda.current_device() == self.device.index:
            return fn(*args)
        with torch.cuda.device(self.device):
            return fn(*args)

    def _check(self, t, shape, what):
        if t.dtype != self.dtype:
            raise TypeError(f"{what} has dtype {t.dtype}, plan expects {self.dtype}")
        if t.device != self.device:
            raise ValueError(f"{what} is on {t.device}, plan is on {self.device}")
        if t.shape != shape:
            raise ValueError(f"{what} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{what} must be contiguous")

    def exchange(self, x, mode: int, chunked: bool = False, out=None, stream=None):
        """Enqueue the exchange on `stream` (default: torch's current stream) and return out."""
        import torch
        self._check(x, self.in_shape(mode), "input")
        if out is None:
            out = torch.empty(self.out_shape(mode), dtype=self.dtype, device=self.device)
        else:
            self._check(out, self.out_shape(mode), "output")
        sptr = _current_raw_stream(self.device) if stream is None else stream.cuda_stream
        handle = self.handle
        args = (handle, mode, int(chunked), x.data_ptr(), out.data_ptr(), sptr or None)
        lib = load_library()
        rc = lib.ua2a_exchange(*args)
        if rc == UA2A_ERR_DEVICE and handle:
            # another device is current: the library changed nothing; retry on the plan's
            with torch.cuda.device(self.device):
                rc = lib.ua2a_exchange(*args)
        if rc != UA2A_OK:
            raise UA2AError(rc, "ua2a_exchange", ua2a_plan_last_error(handle) if handle else "")
        return out

    def exchange_noalloc(self, x, mode: int, out, stream=None):
        """Chunked exchange through the library's own window
        (ua2a_exchange_chunked_noalloc): nothing is allocated, so the caller
        passes `out`; calls that can overlap on one device race on the
        shared window.  Returns out."""
        import torch
        self._check(x, self.in_shape(mode), "input")
        self._check(out, self.out_shape(mode), "output")
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        self._on_device(ua2a_exchange_chunked_noalloc, self.handle, mode, x.data_ptr(), out.data_ptr(),
                        stream.cuda_stream)
        return out

    def _check_ranks(self, xs, outs, mode: int, first: int, count: int) -> None:
        w = self.w
        if len(xs) != w:
            raise ValueError(f"xs needs one entry per rank ({w}), got {len(xs)}")
        if not (0 <= first and 1 <= count and first + count <= w):
            raise ValueError(f"sender range [{first}, {first + count}) is not within [0, {w})")
        for k in range(first, first + count):
            if xs[k] is None:
                raise ValueError(f"sending rank {k} has no input")
            self._check(xs[k], self.in_shape(mode)[1:], f"input of rank {k}")
        if len(outs) != w:
            raise ValueError(f"outs needs one entry per rank ({w}), got {len(outs)}")
        for k, o in enumerate(outs):
            self._check(o, self.out_shape(mode)[1:], f"output of rank {k}")

    def exchange_ranks(self, xs, mode: int, outs=None, first: int = 0, count=None, stream=None):
        """Exchange between per-rank tensors: xs[k] is rank k's input (the
        rank-stacked shape without its leading w), indexed by sending rank;
        only xs[first : first+count] are read and the other entries may be
        None.  Returns outs (allocated with torch.empty when None), indexed by
        receiving rank; only the runs from the senders are written."""
        import torch
        count = self.w - first if count is None else count
        if outs is None:
            outs = [torch.empty(self.out_shape(mode)[1:], dtype=self.dtype, device=self.device)
                    for _ in range(self.w)]
        self._check_ranks(xs, outs, mode, first, count)
        in_ptrs = [None if x is None else x.data_ptr() for x in xs]
        out_ptrs = [o.data_ptr() for o in outs]
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        self._on_device(ua2a_exchange_ranks, self.handle, mode, in_ptrs, out_ptrs, first, count,
                        stream.cuda_stream)
        return outs

    def window_shape(self):
        """Shape of one receiver's window for pack_ranks / unpack_ranks: one
        rank's sequence-gathered tensor, [B, S_local*w, H//w, D]."""
        return (self.B, self.S_local * self.w, self.H // self.w, self.D)

    def pack_ranks(self, xs, mode: int, wins=None, first: int = 0, count=None, stream=None):
        """Senders [first, first+count) write their shares into every
        receiver's window (token block k of each plane holds sender k's share);
        xs as for exchange_ranks.  Returns wins (allocated when None)."""
        import torch
        count = self.w - first if count is None else count
        if wins is None:
            wins = [torch.empty(self.window_shape(), dtype=self.dtype, device=self.device)
                    for _ in range(self.w)]
        if len(wins) != self.w:
            raise ValueError(f"wins needs one entry per rank ({self.w}), got {len(wins)}")
        for q, wn in enumerate(wins):
            self._check(wn, self.window_shape(), f"window of rank {q}")
        if len(xs) != self.w:
            raise ValueError(f"xs needs one entry per rank ({self.w}), got {len(xs)}")
        if not (0 <= first and 1 <= count and first + count <= self.w):
            raise ValueError(f"sender range [{first}, {first + count}) is not within [0, {self.w})")
        for k in range(first, first + count):
            if xs[k] is None:
                raise ValueError(f"sending rank {k} has no input")
            self._check(xs[k], self.in_shape(mode)[1:], f"input of rank {k}")
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        self._on_device(ua2a_pack_ranks, self.handle, mode, [None if x is None else x.data_ptr() for x in xs],
                        [wn.data_ptr() for wn in wins], first, count, stream.cuda_stream)
        return wins

    def unpack_ranks(self, wins, mode: int, outs=None, first: int = 0, count=None, stream=None):
        """Receivers [first, first+count) move their windows into their outputs
        (one launch each).  Returns outs (allocated when None; entries outside
        the range may be None)."""
        import torch
        count = self.w - first if count is None else count
        if not (0 <= first and 1 <= count and first + count <= self.w):
            raise ValueError(f"receiver range [{first}, {first + count}) is not within [0, {self.w})")
        if outs is None:
            outs = [torch.empty(self.out_shape(mode)[1:], dtype=self.dtype, device=self.device)
                    if first <= q < first + count else None for q in range(self.w)]
        if len(wins) != self.w or len(outs) != self.w:
            raise ValueError(f"wins and outs need one entry per rank ({self.w})")
        for q in range(first, first + count):
            self._check(wins[q], self.window_shape(), f"window of rank {q}")
            self._check(outs[q], self.out_shape(mode)[1:], f"output of rank {q}")
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        self._on_device(ua2a_unpack_ranks, self.handle, mode,
                        [None if wn is None else wn.data_ptr() for wn in wins],
                        [None if o is None else o.data_ptr() for o in outs], first, count, stream.cuda_stream)
        return outs

    def bind(self, x, mode: int, chunked: bool = False, out=None, stream=None):
        """Check exchange(x, mode, chunked, out) once (nothing is launched) and
        return a no-argument function that issues it on the current device --
        the same tensors and stream every time -- for loops of small exchanges
        where the per-call checks of exchange() cost more than the launch.  The
        function keeps the tensors and this plan alive, reads the plan's handle
        at every call, and raises UA2AError (invalid argument) once the plan is
        closed; `call.out` is the output tensor."""
        import torch
        self._check(x, self.in_shape(mode), "input")
        if out is None:
            out = torch.empty(self.out_shape(mode), dtype=self.dtype, device=self.device)
        else:
            self._check(out, self.out_shape(mode), "output")
        self.describe(x, mode, chunked, out=out)          # the library's own checks
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        fn = load_library().ua2a_exchange
        xptr, optr, sptr = x.data_ptr(), out.data_ptr(), stream.cuda_stream or None
        ck = int(chunked)
        plan = self

        def call():
            handle = plan.handle
            if not handle:
                raise UA2AError(UA2A_ERR_INVALID_ARG, "ua2a_exchange", "the plan is closed")
            rc = fn(handle, mode, ck, xptr, optr, sptr)
            if rc != UA2A_OK:
                raise UA2AError(rc, "ua2a_exchange", ua2a_plan_last_error(handle))

        call.tensors = (x, out)
        call.out = out
        call.plan = plan
        return call

    def bind_ranks(self, xs, mode: int, outs, first: int = 0, count=None, stream=None):
        """Check a per-rank call once (nothing is launched) and return a
        no-argument function that issues it on the current device -- the same
        tensors, senders and stream every time -- for loops where per-call
        checks would cost more than the launch.  The function keeps the
        tensors and this plan alive, reads the plan's handle at every call,
        and raises UA2AError (invalid argument) once the plan is closed."""
        import torch
        count = self.w - first if count is None else count
        self._check_ranks(xs, outs, mode, first, count)
        self.describe_ranks(xs, outs, mode, first, count)     # the library's own checks
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        lib = load_library()
        in_tab = _table([None if x is None else x.data_ptr() for x in xs])
        out_tab = _table([o.data_ptr() for o in outs])
        sptr = stream.cuda_stream
        plan = self

        def call():
            handle = plan.handle
            if not handle:
                raise UA2AError(UA2A_ERR_INVALID_ARG, "ua2a_exchange_ranks", "the plan is closed")
            rc = lib.ua2a_exchange_ranks(handle, mode, in_tab, out_tab, first, count, sptr)
            if rc != UA2A_OK:
                raise UA2AError(rc, "ua2a_exchange_ranks", ua2a_plan_last_error(handle))

        call.tensors = (list(xs), list(outs))
        call.plan = plan
        return call

    def exchange_publish(self, x, mode: int, credits, out=None, parts=None, stream=None):
        """exchange(x, mode) in `parts` launches (default w) by receiving rank,
        each followed by a readiness credit for its receivers in `credits` (an
        int32/uint32 device tensor of w counters)."""
        import torch
        self._check(x, self.in_shape(mode), "input")
        parts = self.w if parts is None else parts
        if credits.element_size() != 4 or credits.numel() < self.w or not credits.is_contiguous():
            raise ValueError(f"credits must be a contiguous 4-byte integer tensor of >= {self.w} counters")
        if credits.device != self.device:
            raise ValueError(f"credits are on {credits.device}, plan is on {self.device}")
        if out is None:
            out = torch.empty(self.out_shape(mode), dtype=self.dtype, device=self.device)
        else:
            self._check(out, self.out_shape(mode), "output")
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        self._on_device(ua2a_exchange_publish, self.handle, mode, x.data_ptr(), out.data_ptr(),
                        credits.data_ptr(), parts, stream.cuda_stream)
        return out

    def describe_ranks(self, xs, outs, mode: int, first: int = 0, count=None) -> dict:
        """What exchange_ranks(xs, mode, outs, first, count) would launch."""
        count = self.w - first if count is None else count
        return ua2a_describe_ranks(self.handle, mode, [None if x is None else x.data_ptr() for x in xs],
                                   [o.data_ptr() for o in outs], first, count)

    def describe(self, x, mode: int, chunked: bool = False, out=None) -> dict:
        """What exchange(x, mode, chunked, out) would launch.  Without `out`, a
        16-byte-aligned stand-in address past `x` and the window is checked."""
        if out is not None:
            optr = out.data_ptr()
        else:
            end = x.data_ptr() + self.layout["tensor_bytes"]
            if self.window is not None:
                end = max(end, self.window.data_ptr() + self.window.numel() * self.window.element_size())
            optr = (end + 255) // 256 * 256
        return ua2a_describe(self.handle, mode, int(chunked), x.data_ptr(), optr)

    def set_path(self, path: int) -> None:
        ua2a_plan_set_path(self.handle, path)

    def last_error(self) -> str:
        return ua2a_plan_last_error(self.handle)

    def close(self) -> None:
        if getattr(self, "handle", None):
            ua2a_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
