"""Pins of the CPU oracle to facts that the pages and mathematics fix (CPU only).

The FastVideo ``ulysses_a2a`` page (method ``run_armed``) states the shapes
of both modes and the chunked per-plane loop; ``try_all_to_all_4D`` on the
same page falls back to the framework's own all-to-all when the fused path
declines, so the fused exchange must give exactly what that all-to-all gives.
The pins below therefore check the oracle against:

* the closed-form output shapes of both modes;
* w = 1 (nothing to exchange: output bytes equal input bytes);
* mode 1 undoing mode 0 and mode 0 undoing mode 1, byte for byte;
* chunked == unchunked (the chunked branch is the same call per plane);
* a real all-to-all over torch.distributed's gloo backend in w processes
  (the collective's chunk order, not this file, decides where data lands);
* numpy's reshape/transpose view of the same re-layout;
* hand-derived worked examples in tests/golden/hand_examples.json;
* the element multiset (the exchange is a bijection);
* raw bit patterns (NaN payloads, -0.0, denormals) passing unchanged.

``test_pins_reject_plausible_mistakes`` shows that each plausible slip in a
re-layout (interleaved token order, strided head blocks, rank/plane mix-up,
reversed ranks, head/dim swap) fails at least one pin.
"""
from __future__ import annotations

import ctypes
import json
import os
import socket

import numpy as np
import pytest

import oracle
from workloads import CONFIGS, TAIL_SHAPES

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")

# (w, B, S_local, H, D): several tiles' worth of ragged shapes, w from 1 to 6
SHAPES = [
    (2, 1, 8, 4, 16),
    (1, 2, 3, 5, 7),
    (3, 2, 5, 6, 4),
    (4, 3, 7, 8, 3),
    (5, 1, 4, 10, 2),
    (6, 2, 3, 12, 1),
    (2, 2, 3, 6, 5),
]


def rand_bits(shape, itemsize, seed):
    """Uniform random bit patterns, viewed as an unsigned integer of `itemsize` bytes."""
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    raw = rng.integers(0, 256, size=n * itemsize, dtype=np.uint8)
    return raw.view({1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[itemsize]).reshape(shape)


def mode1_shape(w, B, S_local, H, D):
    return (w, B, S_local * w, H // w, D)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("shape", SHAPES)
def test_output_shapes(shape):
    w, B, S, H, D = shape
    x = rand_bits((w, B, S, H, D), 2, 0)
    y = oracle.exchange(x, 0, w)
    assert y.shape == (w, B, S * w, H // w, D)
    z = oracle.exchange(y, 1, w)
    assert z.shape == (w, B, S, H, D)


@pytest.mark.parametrize("itemsize", [1, 2, 4, 8])
@pytest.mark.parametrize("B,S,H,D", [(1, 5, 3, 7), (2, 4, 6, 2), (3, 1, 1, 1)])
def test_w1_is_identity(itemsize, B, S, H, D):
    x = rand_bits((1, B, S, H, D), itemsize, 1)
    for mode in (0, 1):
        for chunked in (False, True):
            y = oracle.exchange(x, mode, 1, chunked=chunked)
            assert y.shape == x.shape
            assert y.tobytes() == x.tobytes()


@pytest.mark.parametrize("itemsize", [1, 2, 4, 8])
@pytest.mark.parametrize("shape", SHAPES)
def test_round_trips(shape, itemsize):
    w, B, S, H, D = shape
    x = rand_bits((w, B, S, H, D), itemsize, 2)
    y = oracle.exchange(x, 0, w)
    assert oracle.exchange(y, 1, w).tobytes() == x.tobytes()
    v = rand_bits(mode1_shape(*shape), itemsize, 3)
    u = oracle.exchange(v, 1, w)
    assert oracle.exchange(u, 0, w).tobytes() == v.tobytes()


@pytest.mark.parametrize("shape", SHAPES + [s[:5] for s in TAIL_SHAPES])
def test_chunked_equals_unchunked(shape):
    w, B, S, H, D = shape
    x = rand_bits((w, B, S, H, D), 2, 4)
    assert oracle.exchange(x, 0, w, chunked=True).tobytes() == oracle.exchange(x, 0, w).tobytes()
    v = rand_bits(mode1_shape(w, B, S, H, D), 4, 5)
    assert oracle.exchange(v, 1, w, chunked=True).tobytes() == oracle.exchange(v, 1, w).tobytes()


@pytest.mark.parametrize("shape", SHAPES)
def test_bijection(shape):
    w, B, S, H, D = shape
    n = w * B * S * H * D
    x = np.arange(n, dtype=np.int64).reshape(w, B, S, H, D)   # every value unique
    for mode, inp in ((0, x), (1, x.reshape(mode1_shape(*shape)))):
        y = oracle.exchange(inp, mode, w)
        assert np.array_equal(np.sort(y.ravel()), np.arange(n))


def test_raw_bits_pass_unchanged():
    w, B, S, H, D = 3, 2, 5, 6, 4
    specials32 = np.array([0x7FC01234, 0xFFC00001, 0x80000000, 0x00000001, 0x7F800000,
                           0xFF800000, 0x007FFFFF, 0x7FA00000], dtype=np.uint32)
    x = np.resize(specials32, (w, B, S, H, D))
    xf = x.view(np.float32)                 # NaN payloads, -0.0, denormals, infinities
    y = oracle.exchange(xf, 0, w)
    z = oracle.exchange(y, 1, w)
    assert z.view(np.uint32).tobytes() == x.tobytes()
    assert np.array_equal(np.sort(y.view(np.uint32).ravel()), np.sort(x.ravel()))


# ----------------------------------------------------------- library routines

def numpy_mode0(x, w):
    """All-to-all as numpy sees it: split heads into w blocks, move the block axis to the front."""
    _, B, S, H, D = x.shape
    Hl = H // w
    t = x.reshape(w, B, S, w, Hl, D)            # [src rank, B, S, dst rank, Hl, D]
    t = t.transpose(3, 1, 0, 2, 4, 5)           # [dst rank, B, src rank, S, Hl, D]
    return t.reshape(w, B, w * S, Hl, D)


def numpy_mode1(y, w):
    _, B, Sg, Hl, D = y.shape
    S = Sg // w
    t = y.reshape(w, B, w, S, Hl, D)            # [head-block owner, B, token owner, S, Hl, D]
    t = t.transpose(2, 1, 3, 0, 4, 5)           # [token owner, B, S, head-block owner, Hl, D]
    return t.reshape(w, B, S, w * Hl, D)


@pytest.mark.parametrize("shape", SHAPES)
def test_matches_numpy_transpose(shape):
    w = shape[0]
    x = rand_bits(shape, 4, 6)
    assert np.array_equal(oracle.exchange(x, 0, w), numpy_mode0(x, w))
    v = rand_bits(mode1_shape(*shape), 4, 7)
    assert np.array_equal(oracle.exchange(v, 1, w), numpy_mode1(v, w))


def test_full_size_awkward_matches_numpy():
    """Five-config awkward shape at full size with unique int32 indices (exact provenance)."""
    c = CONFIGS["awkward"]
    w, B, S, H, D = c["w"], c["B"], c["S_local"], c["H"], c["D"]
    x = np.arange(w * B * S * H * D, dtype=np.int32).reshape(w, B, S, H, D)
    y = oracle.exchange(x, 0, w)
    assert np.array_equal(y, numpy_mode0(x, w))
    assert np.array_equal(oracle.exchange(y, 1, w), x)


# ------------------------------------------------------------- golden examples

def load_golden():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", load_golden(), ids=lambda e: e["name"])
def test_hand_examples(ex):
    w = ex["w"]
    x = np.array(ex["mode0_input"], dtype=np.int32)
    y = np.array(ex["mode0_output"], dtype=np.int32)
    assert x.shape == (w, ex["B"], ex["S_local"], ex["H"], ex["D"])
    assert np.array_equal(oracle.exchange(x, 0, w), y)
    assert np.array_equal(oracle.exchange(y, 1, w), x)
    assert np.array_equal(oracle.exchange(x, 0, w, chunked=True), y)
    assert np.array_equal(oracle.exchange(y, 1, w, chunked=True), x)


# ------------------------------------------- all-to-all over gloo, w processes

def _free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def _gloo_rank(rank, w, port, workdir):
    """One rank: the classic 4-D all-to-all built on all_to_all_single."""
    import torch
    import torch.distributed as dist
    os.environ["MASTER_ADDR"] = "127.0.0.1"
    os.environ["MASTER_PORT"] = str(port)
    dist.init_process_group("gloo", rank=rank, world_size=w)
    try:
        x = torch.from_numpy(np.load(os.path.join(workdir, "x0.npy"))[rank])   # [B,S,H,D]
        B, S, H, D = x.shape
        Hl = H // w
        # mode 0: chunk k of the send buffer is head block k; it goes to rank k
        send = x.reshape(B, S, w, Hl, D).permute(2, 0, 1, 3, 4).contiguous()
        recv = torch.empty_like(send)            # recv[k] = what rank k sent to me
        dist.all_to_all_single(recv, send)
        y = recv.permute(1, 0, 2, 3, 4).reshape(B, w * S, Hl, D)
        np.save(os.path.join(workdir, f"y0_{rank}.npy"), y.numpy())
        # mode 1 on an independent input: chunk k is token block k; it goes to rank k
        v = torch.from_numpy(np.load(os.path.join(workdir, "x1.npy"))[rank])   # [B,Sg,Hl,D]
        send = v.reshape(B, w, S, Hl, D).permute(1, 0, 2, 3, 4).contiguous()
        recv = torch.empty_like(send)            # recv[k] = my tokens, head block k
        dist.all_to_all_single(recv, send)
        u = recv.permute(1, 2, 0, 3, 4).reshape(B, S, w * Hl, D)
        np.save(os.path.join(workdir, f"y1_{rank}.npy"), u.numpy())
    finally:
        dist.destroy_process_group()


def gloo_exchange(x0, x1, w, workdir):
    import torch.multiprocessing as mp
    np.save(os.path.join(workdir, "x0.npy"), x0)
    np.save(os.path.join(workdir, "x1.npy"), x1)
    mp.spawn(_gloo_rank, args=(w, _free_port(), str(workdir)), nprocs=w, join=True)
    y0 = np.stack([np.load(os.path.join(workdir, f"y0_{r}.npy")) for r in range(w)])
    y1 = np.stack([np.load(os.path.join(workdir, f"y1_{r}.npy")) for r in range(w)])
    return y0, y1


@pytest.mark.slow
@pytest.mark.parametrize("shape", [(2, 2, 5, 4, 3), (3, 1, 4, 6, 2), (4, 2, 3, 8, 5)])
def test_matches_gloo_all_to_all(shape, tmp_path):
    w = shape[0]
    n = int(np.prod(shape))
    x0 = np.arange(n, dtype=np.int64).reshape(shape)
    x1 = (np.arange(n, dtype=np.int64) * 7 + 3).reshape(mode1_shape(*shape))
    y0, y1 = gloo_exchange(x0, x1, w, tmp_path)
    assert np.array_equal(oracle.exchange(x0, 0, w), y0)
    assert np.array_equal(oracle.exchange(x1, 1, w), y1)
    assert np.array_equal(oracle.exchange(x0, 0, w, chunked=True), y0)
    # every plausible slip below disagrees with the collective on this input
    # (a rank/plane mix-up cannot show when there is a single plane)
    for name, wrong in MISTAKES.items():
        if name == "rank_plane_mixup" and shape[1] == 1:
            continue
        assert not np.array_equal(wrong(x0, w), y0), name


# ------------------------------------------------- the pins discriminate slips

def _interleaved_tokens(x, w):           # global token = s*w + j instead of j*S + s
    _, B, S, H, D = x.shape
    t = x.reshape(w, B, S, w, H // w, D).transpose(3, 1, 2, 0, 4, 5)
    return t.reshape(w, B, S * w, H // w, D)


def _strided_heads(x, w):                # rank r keeps heads r, r+w, ... instead of a block
    _, B, S, H, D = x.shape
    t = x.reshape(w, B, S, H // w, w, D).transpose(4, 1, 0, 2, 3, 5)
    return t.reshape(w, B, S * w, H // w, D)


def _rank_plane_mixup(x, w):             # reads the stack as [B][w] instead of [w][B]
    _, B, S, H, D = x.shape
    return numpy_mode0(x.reshape(B, w, S, H, D).transpose(1, 0, 2, 3, 4).copy(), w)


def _reversed_ranks(x, w):               # rank r receives head block w-1-r
    return numpy_mode0(x, w)[::-1].copy()


def _head_dim_swap(x, w):                # moves [Hl, D] as [D, Hl]
    y = numpy_mode0(x, w)
    return np.ascontiguousarray(np.swapaxes(y, 3, 4)).reshape(y.shape)


MISTAKES = {
    "interleaved_tokens": _interleaved_tokens,
    "strided_heads": _strided_heads,
    "rank_plane_mixup": _rank_plane_mixup,
    "reversed_ranks": _reversed_ranks,
    "head_dim_swap": _head_dim_swap,
}


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_pins_reject_plausible_mistakes(name):
    wrong = MISTAKES[name]
    caught = []
    for ex in load_golden():
        x = np.array(ex["mode0_input"], dtype=np.int32)
        y = np.array(ex["mode0_output"], dtype=np.int32)
        if not np.array_equal(wrong(x, ex["w"]), y):
            caught.append(ex["name"])
    # the same slip must also break agreement with the oracle on a generic shape
    x = rand_bits((3, 2, 5, 6, 4), 4, 8)
    assert not np.array_equal(wrong(x, 3), oracle.exchange(x, 0, 3)), name
    assert caught, f"{name} passes every hand example"


# --------------------------------------------------------------- argument checks

def test_argument_errors():
    buf = ctypes.create_string_buffer(4096)
    p = ctypes.addressof(buf)
    f = "ua2a_oracle_mode0"
    assert oracle.raw_call(f, 2, 1, 2, 4, 1, 2, p, p + 2048) == 0
    assert oracle.raw_call(f, 2, 1, 2, 4, 1, 3, p, p + 2048) == -1      # elem_bytes
    assert oracle.raw_call(f, 2, 1, 2, 4, 1, 2, None, p) == -1          # null input
    assert oracle.raw_call(f, 2, 1, 2, 3, 1, 2, p, p + 2048) == -2      # H % w != 0
    assert oracle.raw_call(f, 0, 1, 2, 4, 1, 2, p, p + 2048) == -2      # w < 1
    assert oracle.raw_call(f, 2, 0, 2, 4, 1, 2, p, p + 2048) == -2      # B < 1
    assert oracle.raw_call("ua2a_oracle_chunked", 2, 2, 1, 2, 4, 1, 2, p, p + 2048) == -1  # mode 2
    with pytest.raises(oracle.OracleError):
        oracle.exchange(np.zeros((2, 1, 2, 3, 1), np.int16), 0, 2)


# ------------------------------------------------- per-element source index

@pytest.mark.parametrize("shape", SHAPES + [(2, 2, 37, 2, 1024)])
def test_source_index_agrees_with_the_whole_oracle(shape):
    """Every output position, both modes: the element oracle names the input
    position the whole-tensor oracle copied there (index-valued inputs)."""
    w, B, S, H, D = shape
    n = w * B * S * H * D
    for mode, in_shape in ((0, shape), (1, mode1_shape(*shape))):
        x = np.arange(n, dtype=np.int64).reshape(in_shape)
        y = oracle.exchange(x, mode, w).ravel()
        src = oracle.source_indices(mode, w, B, S, H, D, np.arange(n, dtype=np.int64))
        assert np.array_equal(src, y)


def test_source_index_rejects_out_of_range():
    assert oracle.raw_call("ua2a_oracle_source_index", 0, 2, 1, 8, 4, 16, 2 * 8 * 4 * 16) == -1
    assert oracle.raw_call("ua2a_oracle_source_index", 0, 2, 1, 8, 4, 16, -1) == -1
    assert oracle.raw_call("ua2a_oracle_source_index", 2, 2, 1, 8, 4, 16, 0) == -1
    assert oracle.raw_call("ua2a_oracle_source_index", 0, 2, 1, 8, 3, 16, 0) == -1
    with pytest.raises(oracle.OracleError):
        oracle.source_indices(0, 2, 1, 8, 4, 16, np.array([5000], dtype=np.int64))


# ------------------------------------------------- per-rank allocations

@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape", SHAPES)
def test_ranks_sender_ranges_match_masked_numpy(shape, mode):
    """Per-rank form, every sender range: an output element holds the numpy
    permutation's value when the rank it comes from is a sender, else its
    fill is untouched.  Index-valued inputs name each element's source rank
    (value // elements per rank); non-senders' inputs are passed as None."""
    w, B, S, H, D = shape
    n = w * B * S * H * D
    in_shape = shape if mode == 0 else mode1_shape(*shape)
    x = np.arange(n, dtype=np.int64).reshape(in_shape)
    full = numpy_mode0(x, w) if mode == 0 else numpy_mode1(x, w)
    src_rank = full // (n // w)
    for first in range(w):
        for count in range(1, w - first + 1):
            xs = [x[k].copy() if first <= k < first + count else None for k in range(w)]
            outs = [np.full(full.shape[1:], -1, np.int64) for _ in range(w)]
            oracle.exchange_ranks(xs, outs, mode, first, count)
            sel = (src_rank >= first) & (src_rank < first + count)
            assert np.array_equal(np.stack(outs), np.where(sel, full, -1)), (first, count)


@pytest.mark.parametrize("itemsize", [1, 2, 4, 8])
@pytest.mark.parametrize("shape", SHAPES + [s[:5] for s in TAIL_SHAPES])
def test_ranks_single_senders_compose_the_whole_exchange(shape, itemsize):
    """One call per sending rank, each writing only its own runs, together
    give the numpy permutation (random bits, every dtype size)."""
    w = shape[0]
    for mode, in_shape in ((0, shape), (1, mode1_shape(*shape))):
        x = rand_bits(in_shape, itemsize, 8 + mode)
        full = numpy_mode0(x, w) if mode == 0 else numpy_mode1(x, w)
        outs = [np.zeros(full.shape[1:], x.dtype) for _ in range(w)]
        for j in range(w):
            oracle.exchange_ranks([x[k].copy() for k in range(w)], outs, mode, j, 1)
        assert np.array_equal(np.stack(outs), full)


def test_ranks_argument_errors():
    w = 2
    x = [np.zeros((1, 2, 4, 3), np.int16) for _ in range(w)]
    o = [np.zeros((1, 4, 2, 3), np.int16) for _ in range(w)]
    oracle.exchange_ranks(x, o, 0, 0, 2)
    vp = ctypes.c_void_p
    ins = (vp * 2)(x[0].ctypes.data, x[1].ctypes.data)
    outs = (vp * 2)(o[0].ctypes.data, o[1].ctypes.data)
    nulls = (vp * 2)(None, None)
    f = "ua2a_oracle_ranks"
    i, q = ctypes.cast(ins, vp), ctypes.cast(outs, vp)
    assert oracle.raw_call(f, 0, 2, 1, 2, 4, 3, 2, i, q, 0, 2) == 0
    assert oracle.raw_call(f, 2, 2, 1, 2, 4, 3, 2, i, q, 0, 2) == -1     # mode
    assert oracle.raw_call(f, 0, 2, 1, 2, 4, 3, 3, i, q, 0, 2) == -1     # elem_bytes
    assert oracle.raw_call(f, 0, 2, 1, 2, 4, 3, 2, i, q, 1, 2) == -1     # first + count > w
    assert oracle.raw_call(f, 0, 2, 1, 2, 4, 3, 2, i, q, 0, 0) == -1     # count < 1
    assert oracle.raw_call(f, 0, 2, 1, 2, 4, 3, 2, ctypes.cast(nulls, vp), q, 0, 1) == -1   # sender NULL
    assert oracle.raw_call(f, 0, 2, 1, 2, 4, 3, 2, i, ctypes.cast(nulls, vp), 0, 1) == -1   # output NULL
    assert oracle.raw_call(f, 0, 2, 1, 2, 3, 3, 2, i, q, 0, 2) == -2     # H % w
    assert oracle.raw_call(f, 0, 2, 1, 2, 4, 3, 2, None, q, 0, 2) == -1  # no table


# ------------------------------------------- pack and unpack through windows
#
# Receiver q's window is [B, S_local*w, H//w, D]; its token block k of each
# plane holds what sender k sends q.  Each pin restates that with numpy
# slicing and transposes of the rank tensors, independent of the loops.

def numpy_window(x, w, mode, q):
    """Receiver q's whole window from the rank-stacked input x."""
    if mode == 0:                               # x [w, B, S, H, D]: head block q of every sender
        _, B, S, H, D = x.shape
        Hl = H // w
        blk = x[:, :, :, q * Hl:(q + 1) * Hl, :]             # [k, B, S, Hl, D]
    else:                                       # x [w, B, S*w, Hl, D]: token block q of every sender
        _, B, Sg, Hl, D = x.shape
        S = Sg // w
        blk = x[:, :, q * S:(q + 1) * S, :, :]               # [k, B, S, Hl, D]
    k, B, S, Hl, D = blk.shape
    return blk.transpose(1, 0, 2, 3, 4).reshape(B, k * S, Hl, D)


def numpy_unpack(win, w, mode):
    if mode == 0:
        return win.copy()
    B, Sg, Hl, D = win.shape
    S = Sg // w
    return win.reshape(B, w, S, Hl, D).transpose(0, 2, 1, 3, 4).reshape(B, S, w * Hl, D)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape", SHAPES)
def test_pack_sender_ranges_match_numpy_slices(shape, mode):
    """Every sender range: the senders' token blocks of every window hold
    numpy's slices of their tensors, every other block keeps its fill."""
    w, B, S, H, D = shape
    in_shape = shape if mode == 0 else mode1_shape(*shape)
    x = rand_bits(in_shape, 4, 20 + mode)
    wshape = (B, S * w, H // w, D)
    for first in range(w):
        for count in range(1, w - first + 1):
            xs = [x[k].copy() if first <= k < first + count else None for k in range(w)]
            wins = [np.full(wshape, 0xA5A5A5A5, np.uint32) for _ in range(w)]
            oracle.pack_ranks(xs, wins, mode, first, count)
            for q in range(w):
                want = numpy_window(x, w, mode, q).reshape(B, w, S, H // w, D)
                got = wins[q].reshape(B, w, S, H // w, D)
                assert np.array_equal(got[:, first:first + count], want[:, first:first + count]), (q, first, count)
                rest = np.concatenate([got[:, :first], got[:, first + count:]], axis=1)
                assert (rest == 0xA5A5A5A5).all(), (q, first, count)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape", SHAPES)
def test_unpack_receiver_ranges_match_numpy_transpose(shape, mode):
    w, B, S, H, D = shape
    wins = [rand_bits((B, S * w, H // w, D), 2, 30 + q) for q in range(w)]
    out_shape = (B, S * w, H // w, D) if mode == 0 else (B, S, H, D)
    for first in range(w):
        for count in range(1, w - first + 1):
            outs = [np.full(out_shape, 7, np.uint16) if first <= q < first + count else None for q in range(w)]
            oracle.unpack_ranks(wins, outs, mode, first, count)
            for q in range(first, first + count):
                assert np.array_equal(outs[q], numpy_unpack(wins[q], w, mode)), (q, first, count)


@pytest.mark.parametrize("itemsize", [1, 2, 4, 8])
@pytest.mark.parametrize("shape", SHAPES + [s[:5] for s in TAIL_SHAPES])
def test_pack_then_unpack_is_the_exchange(shape, itemsize):
    """One pack per sender, then one unpack per receiver, gives numpy's
    exchange (itself pinned to a real all-to-all above)."""
    w, B, S, H, D = shape
    for mode, in_shape in ((0, shape), (1, mode1_shape(*shape))):
        x = rand_bits(in_shape, itemsize, 40 + mode)
        full = numpy_mode0(x, w) if mode == 0 else numpy_mode1(x, w)
        wins = [np.zeros((B, S * w, H // w, D), x.dtype) for _ in range(w)]
        for k in range(w):
            oracle.pack_ranks([x[j].copy() for j in range(w)], wins, mode, k, 1)
        outs = [np.zeros(full.shape[1:], x.dtype) for _ in range(w)]
        for q in range(w):
            oracle.unpack_ranks(wins, outs, mode, q, 1)
        assert np.array_equal(np.stack(outs), full), mode


def test_pack_pins_reject_plausible_mistakes():
    """A window built with the senders reversed, with the receiver's block of
    the wrong side (heads where tokens are meant), or an unpack that keeps
    [k][s] order, all disagree with the oracle on a generic shape."""
    w, B, S, H, D = 3, 2, 5, 6, 4
    x0 = rand_bits((w, B, S, H, D), 4, 50)
    x1 = rand_bits(mode1_shape(w, B, S, H, D), 4, 51)
    wins0 = [np.zeros((B, S * w, H // w, D), np.uint32) for _ in range(w)]
    wins1 = [np.zeros((B, S * w, H // w, D), np.uint32) for _ in range(w)]
    oracle.pack_ranks([x0[k].copy() for k in range(w)], wins0, 0)
    oracle.pack_ranks([x1[k].copy() for k in range(w)], wins1, 1)
    # senders reversed
    assert not np.array_equal(wins0[1], numpy_window(x0[::-1].copy(), w, 0, 1))
    # mode 1 taking the token block of the sender instead of the receiver
    wrong = np.stack([x1[k][:, k * S:(k + 1) * S] for k in range(w)], 1).reshape(B, S * w, H // w, D)
    assert not np.array_equal(wins1[1], wrong)
    # unpack in [k][s] order instead of [s][k]
    outs = [np.zeros((B, S, H, D), np.uint32) for _ in range(w)]
    oracle.unpack_ranks(wins1, outs, 1)
    assert not np.array_equal(outs[1], wins1[1].reshape(B, S, H, D))
    assert np.array_equal(outs[1], numpy_unpack(wins1[1], w, 1))


def test_pack_unpack_argument_errors():
    w = 2
    x = [np.zeros((1, 2, 4, 3), np.int16) for _ in range(w)]
    wn = [np.zeros((1, 4, 2, 3), np.int16) for _ in range(w)]
    vp = ctypes.c_void_p
    i = ctypes.cast((vp * 2)(x[0].ctypes.data, x[1].ctypes.data), vp)
    q = ctypes.cast((vp * 2)(wn[0].ctypes.data, wn[1].ctypes.data), vp)
    nulls = ctypes.cast((vp * 2)(None, None), vp)
    for f in ("ua2a_oracle_pack_ranks", "ua2a_oracle_unpack_ranks"):
        assert oracle.raw_call(f, 0, 2, 1, 2, 4, 3, 2, i, q, 0, 2) == 0
        assert oracle.raw_call(f, 2, 2, 1, 2, 4, 3, 2, i, q, 0, 2) == -1     # mode
        assert oracle.raw_call(f, 0, 2, 1, 2, 4, 3, 3, i, q, 0, 2) == -1     # elem_bytes
        assert oracle.raw_call(f, 0, 2, 1, 2, 4, 3, 2, i, q, 1, 2) == -1     # first + count > w
        assert oracle.raw_call(f, 0, 2, 1, 2, 3, 3, 2, i, q, 0, 2) == -2     # H % w
        assert oracle.raw_call(f, 0, 2, 1, 2, 4, 3, 2, nulls, q, 0, 1) == -1  # a used input NULL
        assert oracle.raw_call(f, 0, 2, 1, 2, 4, 3, 2, i, nulls, 0, 1) == -1  # a used output NULL
