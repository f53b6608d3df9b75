"""PyTorch operator over the exchange: autograd, the 4-D all-to-all API, torch.compile.

The FastVideo ``ulysses_a2a`` API page exposes the exchange as
``try_all_to_all_4D(x, scatter_dim, gather_dim)`` and wraps it in an
autograd function.  Here the same entry point works on the rank-stacked
tensors of this library (all ``w`` virtual ranks in one tensor, rank axis
first), and the dims name axes of one rank's 4-D tensor ``[B, S, H, D]``:

    scatter_dim=2, gather_dim=1  -> mode 0 (scatter heads, gather sequence)
    scatter_dim=1, gather_dim=2  -> mode 1 (the inverse)

The exchange is a permutation of elements, so its gradient is the inverse
permutation: the backward of mode m is the exchange in mode 1 - m, run by
the same HIP kernels.  The operator is registered with ``torch.library`` and
has a shape-only fake implementation, so ``torch.compile`` traces it as one
opaque call (where the page has to decline inside compiled regions, this
operator needs no decline).  Every call runs the HIP library; there is no
other implementation.

``chunked=True`` runs the page's chunked form: one batch plane at a time
through a window sized for one plane of every rank.  As the page's
communicator keeps one registered window and rebuilds it larger when a call
needs more (and says so in its log), the operator keeps one window per device
and stream, grows it (never shrinks it) when a larger shape arrives, logs the
growth, and rebuilds the chunked plans that borrowed the old one.  Calls on
one stream share its window in stream order; other streams get windows of
their own.

Both caches are bounded: at most ``MAX_PLANS`` plans and ``MAX_WINDOWS``
windows are kept, the least recently used going first (a window's plans go
with it).  A dropped window returns to torch's allocator in its own stream's
order, after the work already queued there.  One lock covers the lookup and
the enqueue of each call, so a plan is never closed while another thread is
between finding it and launching on it.
"""
from __future__ import annotations

import logging
import threading
from collections import OrderedDict

import torch

from . import Plan

MAX_PLANS = 64
MAX_WINDOWS = 8

_log = logging.getLogger(__name__)
_plans: "OrderedDict" = OrderedDict()     # key -> Plan, least recently used first
_windows: "OrderedDict" = OrderedDict()   # (device, stream id) -> uint8 window of chunked exchanges
_lock = threading.Lock()


def _drop_plans_of(win) -> None:
    for k in [k for k, p in _plans.items() if p.window is win]:
        _plans.pop(k).close()


def _window_for(device, stream, nbytes: int):
    """The stream's window, grown to at least nbytes; growing closes the plans
    that borrowed the old one (caller holds _lock)."""
    key = (device, stream.stream_id)
    win = _windows.get(key)
    if win is not None and win.numel() >= nbytes:
        _windows.move_to_end(key)
        return win
    if win is not None:
        _drop_plans_of(win)
        _log.info("ua2a: chunked window of %s stream %d grown from %d to %d bytes",
                  device, stream.stream_id, win.numel(), nbytes)
    else:
        _log.info("ua2a: chunked window of %s stream %d created with %d bytes",
                  device, stream.stream_id, nbytes)
    # the old window is released to torch's allocator in this stream's order
    win = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _windows[key] = win
    _windows.move_to_end(key)
    while len(_windows) > MAX_WINDOWS:
        _, old = _windows.popitem(last=False)
        _drop_plans_of(old)
    return win


def _plan_for(w: int, B: int, S_local: int, H: int, D: int, dtype, device,
              chunked: bool = False) -> Plan:
    """One cached plan per shape, dtype and device (plans are small host
    objects); chunked plans per stream too, each borrowing its stream's
    window (caller holds _lock)."""
    window = None
    key = (w, B, S_local, H, D, dtype, device)
    if chunked:
        stream = torch.cuda.current_stream(device)
        e = torch.empty((), dtype=dtype).element_size()
        need = Plan.window_bytes(w, B, S_local, H, D, e)
        window = _window_for(device, stream, need)
        key += (stream.stream_id,)
    plan = _plans.get(key)
    if plan is None:
        plan = Plan(w, B, S_local, H, D, dtype, window=window, device=device)
        _plans[key] = plan
        while len(_plans) > MAX_PLANS:
            _plans.popitem(last=False)[1].close()
    else:
        _plans.move_to_end(key)
    return plan


def _local_shape(shape, w: int, mode: int):
    """(B, S_local, H, D) of a rank-stacked input of the given mode."""
    if len(shape) != 5 or shape[0] != w:
        raise ValueError(f"expected a rank-stacked [w={w}, B, S, H, D] tensor, got {tuple(shape)}")
    _, B, S, Hx, D = shape
    if mode == 0:
        return B, S, Hx, D
    if S % w:
        raise ValueError(f"mode 1 needs S_global = {S} divisible by w = {w}")
    return B, S // w, Hx * w, D


def _out_shape(shape, w: int, mode: int):
    B, S, H, D = _local_shape(shape, w, mode)
    if H % w:
        raise ValueError(f"H = {H} is not divisible by w = {w}")
    return (w, B, S * w, H // w, D) if mode == 0 else (w, B, S, H, D)


@torch.library.custom_op("ua2a::exchange", mutates_args=())
def exchange(x: torch.Tensor, w: int, mode: int, chunked: bool = False) -> torch.Tensor:
    """Rank-stacked Ulysses exchange on the GPU (mode 0 or 1); returns a new tensor."""
    if mode not in (0, 1):
        raise ValueError("mode must be 0 or 1")
    if x.device.type != "cuda":
        raise RuntimeError(f"the exchange runs on the GPU only (got a {x.device.type} tensor)")
    B, S, H, D = _local_shape(x.shape, w, mode)
    x = x.contiguous()
    with _lock:
        plan = _plan_for(w, B, S, H, D, x.dtype, x.device, chunked)
        return plan.exchange(x, mode, chunked)


@exchange.register_fake
def _exchange_fake(x: torch.Tensor, w: int, mode: int, chunked: bool = False) -> torch.Tensor:
    return x.new_empty(_out_shape(x.shape, w, mode))


def _setup_context(ctx, inputs, output):
    _, w, mode, chunked = inputs
    ctx.w = w
    ctx.mode = mode
    ctx.chunked = chunked


def _backward(ctx, grad):
    # d(out)/d(in) is a permutation matrix; its transpose is the inverse exchange
    return exchange(grad.contiguous(), ctx.w, 1 - ctx.mode, ctx.chunked), None, None, None


exchange.register_autograd(_backward, setup_context=_setup_context)


def all_to_all_4D(x: torch.Tensor, scatter_dim: int, gather_dim: int, w: int,
                  chunked: bool = False) -> torch.Tensor:
    """The page's 4-D all-to-all on rank-stacked tensors ``[w, B, S, H, D]``.

    ``scatter_dim`` / ``gather_dim`` index one rank's ``[B, S, H, D]``: (2, 1)
    scatters heads and gathers the sequence (mode 0), (1, 2) is the inverse
    (mode 1).  Other pairs are not an exchange this operator implements.
    ``chunked`` moves one batch plane at a time through the stream's window.
    """
    if (scatter_dim, gather_dim) == (2, 1):
        mode = 0
    elif (scatter_dim, gather_dim) == (1, 2):
        mode = 1
    else:
        raise ValueError(f"unsupported (scatter_dim, gather_dim) = ({scatter_dim}, {gather_dim}); "
                         "use (2, 1) for heads -> sequence or (1, 2) for the inverse")
    return exchange(x, w, mode, chunked)
