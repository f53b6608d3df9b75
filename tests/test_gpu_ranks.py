"""GPU parity of the per-rank exchange (ua2a_exchange_ranks) and of its two-step
form through receive windows (ua2a_pack_ranks, ua2a_unpack_ranks) against
the CPU oracle.

Each rank's input and output is a tensor of its own (a separate device
allocation); outputs start poisoned so that the runs of non-sending ranks
can be checked to stay untouched.  Byte-for-byte comparisons throughout.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import ulysses_all_re_amd as ua
from workloads import BITS_VIEW, CONFIGS, TAIL_SHAPES, make_tensor

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32,
          "f64": torch.float64, "u8": torch.uint8}


def note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ua.load_library()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def bits(t):
    return t.view(BITS_VIEW[t.element_size()])


def poison_bits(dtype):
    return 255 if torch.empty((), dtype=dtype).element_size() == 1 else -1


def stacked_shapes(w, B, S, H, D, mode):
    a, b = (w, B, S, H, D), (w, B, S * w, H // w, D)
    return (a, b) if mode == 0 else (b, a)


def run_case(plan, x_stacked, mode, first, count, offsets=None):
    """Per-rank exchange of the ranks of `x_stacked` (CPU) on the device;
    returns (device outputs as CPU bit tensors, oracle outputs)."""
    w = plan.w
    dt = x_stacked.dtype
    ish, osh = stacked_shapes(plan.w, plan.B, plan.S_local, plan.H, plan.D, mode)
    pb = poison_bits(dt)
    if offsets is None:
        xs = [x_stacked[k].to(DEV) if first <= k < first + count else None for k in range(w)]
        outs = []
        for _ in range(w):
            o = torch.empty(osh[1:], dtype=dt, device=DEV)
            bits(o).fill_(pb)
            outs.append(o)
    else:
        # every rank's tensors at its own element offset inside a larger allocation
        n = int(np.prod(ish[1:]))
        xs, outs = [], []
        for k in range(w):
            oi, oo = offsets[k]
            if first <= k < first + count:
                buf = torch.empty(n + oi, dtype=dt, device=DEV)
                buf[oi:].copy_(x_stacked[k].reshape(-1).to(DEV))
                xs.append(buf[oi:].view(ish[1:]))
            else:
                xs.append(None)
            ob = torch.empty(n + oo, dtype=dt, device=DEV)
            bits(ob).fill_(pb)
            outs.append(ob[oo:].view(osh[1:]))
    plan.exchange_ranks(xs, mode, outs=outs, first=first, count=count)
    torch.cuda.synchronize()
    got = [bits(o.cpu()) for o in outs]
    xb = bits(x_stacked).numpy()
    want = [np.full(osh[1:], pb, dtype=xb.dtype) for _ in range(w)]
    oracle.exchange_ranks([xb[k] if first <= k < first + count else None for k in range(w)],
                          want, mode, first, count)
    return got, [torch.from_numpy(a) for a in want]


def assert_ranks_equal(got, want, what):
    for k, (g, t) in enumerate(zip(got, want)):
        if not torch.equal(g, t):
            bad = (g != t).nonzero()
            raise AssertionError(f"{what}: rank {k}: {bad.shape[0]} elements differ; first at {bad[0].tolist()}")


@pytest.mark.parametrize("name", ["tiny", "mid", "video_dit", "chunked", "awkward"])
def test_workload_ranks_parity(name):
    """Each workload, both modes: the whole exchange (all senders), the first
    and last sender alone, and every sender one call at a time."""
    c = CONFIGS[name]
    w, B, S, H, D = c["w"], c["B"], c["S_local"], c["H"], c["D"]
    dt = DTYPES[c["dtype"]]
    plan = ua.Plan(w, B, S, H, D, dt)
    for mode in (0, 1):
        ish, _ = stacked_shapes(w, B, S, H, D, mode)
        dist = c["dist"] if (c["dist"] != "index" or mode == 0) else "index_bits"
        x = make_tensor(ish, c["dtype"], dist, c["seed0"] if mode == 0 else c["seed1"])
        for first, count in ((0, w), (0, 1), (w - 1, 1)):
            note(f"ranks {name} mode{mode} senders=[{first},{first + count}) shape={tuple(ish)}")
            got, want = run_case(plan, x, mode, first, count)
            assert_ranks_equal(got, want, f"{name} mode {mode} senders [{first}, {first + count})")
        # one call per sender into the same outputs gives the whole exchange
        note(f"ranks {name} mode{mode} composed from single senders")
        _, osh = stacked_shapes(w, B, S, H, D, mode)
        xs = [x[k].to(DEV) for k in range(w)]
        outs = [torch.zeros(osh[1:], dtype=dt, device=DEV) for _ in range(w)]
        for j in range(w):
            plan.exchange_ranks(xs, mode, outs=outs, first=j, count=1)
        whole = plan.exchange_ranks(xs, mode)
        torch.cuda.synchronize()
        for k in range(w):
            assert torch.equal(bits(outs[k]), bits(whole[k])), (name, mode, k)
        del xs, outs, whole
    plan.close()


@pytest.mark.parametrize("shape", TAIL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ranks_tail_shapes(shape):
    w, B, S, H, D, dname = shape
    dt = DTYPES[dname]
    plan = ua.Plan(w, B, S, H, D, dt)
    for mode in (0, 1):
        ish, _ = stacked_shapes(w, B, S, H, D, mode)
        x = make_tensor(ish, dname, "bytes", 11 + mode)
        for first, count in ((0, w), (w - 1, 1)):
            note(f"ranks tail {shape} mode{mode} senders=[{first},{first + count})")
            got, want = run_case(plan, x, mode, first, count)
            assert_ranks_equal(got, want, f"tail {shape} mode {mode}")
    plan.close()


@pytest.mark.parametrize("shape", [(4, 1, 1024, 24, 128, "bf16"), (3, 1, 5, 3, 7, "bf16"),
                                   (8, 1, 300, 40, 128, "bf16"), (2, 2, 9, 6, 5, "fp32")],
                         ids=lambda s: "x".join(map(str, s)))
def test_ranks_misaligned_bases(shape):
    """Per-rank tensors at different element offsets from their allocations."""
    w, B, S, H, D, dname = shape
    dt = DTYPES[dname]
    plan = ua.Plan(w, B, S, H, D, dt)
    offsets = [((k % 3) + 1, (2 * k + 1) % 5) for k in range(w)]
    for mode in (0, 1):
        ish, _ = stacked_shapes(w, B, S, H, D, mode)
        x = make_tensor(ish, dname, "bytes", 21 + mode)
        note(f"ranks misaligned {shape} mode{mode}")
        got, want = run_case(plan, x, mode, 0, w, offsets)
        assert_ranks_equal(got, want, f"misaligned {shape} mode {mode}")
    plan.close()


def _random_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        w = int(rng.integers(1, 17))
        hl = int(rng.integers(1, 6))
        D = int(rng.choice([1, 3, 8, 16, 40, 64, 80, 128, 129]))
        B = int(rng.integers(1, 4))
        S = int(rng.integers(1, 700))
        dname = str(rng.choice(["bf16", "fp32", "u8", "f64"]))
        mode = int(rng.integers(0, 2))
        first = int(rng.integers(0, w))
        count = int(rng.integers(1, w - first + 1))
        cases.append((w, B, S, w * hl, D, dname, mode, first, count))
    return cases


@pytest.mark.parametrize("case", _random_cases(30, 77), ids=lambda c: "x".join(map(str, c)))
def test_ranks_random_cases(case):
    w, B, S, H, D, dname, mode, first, count = case
    dt = DTYPES[dname]
    plan = ua.Plan(w, B, S, H, D, dt)
    ish, _ = stacked_shapes(w, B, S, H, D, mode)
    x = make_tensor(ish, dname, "bytes", sum(case[:5]))
    note(f"ranks random {case}")
    got, want = run_case(plan, x, mode, first, count)
    assert_ranks_equal(got, want, f"random {case}")
    plan.close()


def test_ranks_largest_table():
    w = 64
    plan = ua.Plan(w, 1, 33, 64, 16, torch.bfloat16)
    for mode in (0, 1):
        ish, _ = stacked_shapes(w, 1, 33, 64, 16, mode)
        x = make_tensor(ish, "bf16", "bytes", 31 + mode)
        for first, count in ((0, 64), (40, 9)):
            note(f"ranks w=64 mode{mode} senders=[{first},{first + count})")
            got, want = run_case(plan, x, mode, first, count)
            assert_ranks_equal(got, want, f"w=64 mode {mode}")
    plan.close()


def test_ranks_argument_checks_on_device_tensors():
    plan = ua.Plan(2, 1, 8, 4, 16, torch.bfloat16)
    xs = [torch.zeros(1, 8, 4, 16, dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    with pytest.raises(TypeError):
        plan.exchange_ranks([x.float() for x in xs], 0)
    with pytest.raises(ValueError):
        plan.exchange_ranks(xs[:1], 0)
    with pytest.raises(ValueError):
        plan.exchange_ranks([xs[0], None], 0)
    with pytest.raises(ValueError):
        plan.exchange_ranks(xs, 0, first=1, count=2)
    outs = [torch.empty(1, 16, 2, 16, dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    with pytest.raises(ua.UA2AError) as e:
        plan.exchange_ranks(xs, 0, outs=[outs[0], outs[0]])
    assert e.value.code == ua.UA2A_ERR_ALIAS
    with pytest.raises(ua.UA2AError) as e:
        plan.exchange_ranks(xs, 0, outs=[outs[0], xs[1].view(1, 16, 2, 16)])
    assert e.value.code == ua.UA2A_ERR_ALIAS
    # a non-sender's input is neither read nor checked
    plan.exchange_ranks([xs[0], None], 0, outs=outs, first=0, count=1)
    torch.cuda.synchronize()
    plan.close()


def test_per_rank_exchange_in_a_hip_graph():
    """Capture one sender's per-rank exchange and the whole one; replays with
    new inputs copied in between give the oracle's bytes each time."""
    c = CONFIGS["mid"]
    w, B, S, H, D = c["w"], c["B"], c["S_local"], c["H"], c["D"]
    plan = ua.Plan(w, B, S, H, D, torch.bfloat16)
    ish, osh = stacked_shapes(w, B, S, H, D, 0)
    xs = [torch.zeros(ish[1:], dtype=torch.bfloat16, device=DEV) for _ in range(w)]
    outs = [torch.empty(osh[1:], dtype=torch.bfloat16, device=DEV) for _ in range(w)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.exchange_ranks(xs, 0, outs=outs, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    note("graph capture of per-rank exchanges")
    with torch.cuda.graph(graph):
        plan.exchange_ranks(xs, 0, outs=outs, first=w - 1, count=1)
        plan.exchange_ranks(xs, 0, outs=outs, first=0, count=w - 1)
    for i in range(3):
        x = make_tensor(ish, "bf16", "bytes", 400 + i)
        for k in range(w):
            xs[k].copy_(x[k].to(DEV))
            bits(outs[k]).fill_(-1)
        torch.cuda.synchronize()
        note(f"per-rank graph replay {i}")
        graph.replay()
        torch.cuda.synchronize()
        want = oracle.exchange(bits(x).numpy(), 0, w)
        for k in range(w):
            assert torch.equal(bits(outs[k].cpu()), torch.from_numpy(want[k])), (i, k)
    plan.close()


@pytest.mark.parametrize("blocks", [5, 3000])
def test_ranks_with_a_capped_grid(blocks):
    """A `blocks` cap shrinks the per-rank grid; the kernel's loops cover the rest."""
    w, B, S, H, D = 4, 2, 300, 8, 64
    plan = ua.Plan(w, B, S, H, D, torch.bfloat16, blocks=blocks)
    for mode in (0, 1):
        ish, _ = stacked_shapes(w, B, S, H, D, mode)
        x = make_tensor(ish, "bf16", "bytes", 600 + mode)
        for first, count in ((0, w), (1, 2)):
            note(f"ranks blocks={blocks} mode{mode} senders=[{first},{first + count})")
            got, want = run_case(plan, x, mode, first, count)
            assert_ranks_equal(got, want, f"blocks {blocks} mode {mode} [{first}, {first + count})")
    plan.close()


# ------------------------------------------------- pack and unpack (windows)

def run_pack_unpack(plan, x_stacked, mode, senders, receivers, offsets=None):
    """Pack the senders (one call each) into every receiver's window, then
    unpack the receivers (one call each).  Windows and outputs start
    poisoned; each rank's tensors may sit at an element offset inside a larger
    allocation (offsets[k] = (input, window, output)).  Returns the device
    windows and outputs and the oracle's, all as CPU bit arrays."""
    w = plan.w
    dt = x_stacked.dtype
    ish, osh = stacked_shapes(plan.w, plan.B, plan.S_local, plan.H, plan.D, mode)
    wsh = plan.window_shape()
    pb = poison_bits(dt)
    n = int(np.prod(ish[1:]))
    offsets = offsets or [(0, 0, 0)] * w

    def at(k, which, shape, fill=None, src=None):
        off = offsets[k][which]
        buf = torch.empty(n + off, dtype=dt, device=DEV)
        if fill is not None:
            bits(buf).fill_(fill)
        if src is not None:
            buf[off:].copy_(src.reshape(-1).to(DEV))
        return buf[off:].view(shape)

    used = sorted(set(senders))
    xs = [at(k, 0, ish[1:], src=x_stacked[k]) if k in used else None for k in range(w)]
    wins = [at(k, 1, wsh, fill=pb) for k in range(w)]
    outs = [at(k, 2, osh[1:], fill=pb) for k in range(w)]
    for k in senders:
        plan.pack_ranks(xs, mode, wins, first=k, count=1)
    for q in receivers:
        plan.unpack_ranks(wins, mode, outs, first=q, count=1)
    torch.cuda.synchronize()
    xb = bits(x_stacked).numpy()
    want_w = [np.full(wsh, pb, dtype=xb.dtype) for _ in range(w)]
    for k in senders:
        oracle.pack_ranks([xb[j] if j in used else None for j in range(w)], want_w, mode, k, 1)
    want_o = [np.full(osh[1:], pb, dtype=xb.dtype) for _ in range(w)]
    for q in receivers:
        oracle.unpack_ranks(want_w, want_o, mode, q, 1)
    return ([bits(t.cpu()) for t in wins], [torch.from_numpy(a) for a in want_w],
            [bits(t.cpu()) for t in outs], [torch.from_numpy(a) for a in want_o])


@pytest.mark.parametrize("name", ["tiny", "mid", "video_dit", "chunked", "awkward"])
def test_workload_pack_unpack_parity(name):
    """Each workload, both modes: every sender packs on its own (what one
    device of a multi-device exchange runs), every receiver unpacks on its
    own; windows and outputs equal the oracle's, and the outputs equal the
    oracle's exchange."""
    c = CONFIGS[name]
    w, B, S, H, D = c["w"], c["B"], c["S_local"], c["H"], c["D"]
    dt = DTYPES[c["dtype"]]
    plan = ua.Plan(w, B, S, H, D, dt)
    for mode in (0, 1):
        ish, _ = stacked_shapes(w, B, S, H, D, mode)
        dist = c["dist"] if (c["dist"] != "index" or mode == 0) else "index_bits"
        x = make_tensor(ish, c["dtype"], dist, c["seed0"] if mode == 0 else c["seed1"])
        note(f"pack/unpack {name} mode {mode}")
        gw, ww, go, wo = run_pack_unpack(plan, x, mode, list(range(w)), list(range(w)))
        assert_ranks_equal(gw, ww, f"{name} mode {mode} windows")
        assert_ranks_equal(go, wo, f"{name} mode {mode} outputs")
        full = oracle.exchange(bits(x).numpy(), mode, w)
        assert torch.equal(torch.stack(go), torch.from_numpy(full)), f"{name} mode {mode} exchange"
        del x, gw, ww, go, wo
    plan.close()


@pytest.mark.parametrize("path", ["auto", "lds"])
@pytest.mark.parametrize("shape", TAIL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_tail_pack_unpack_parity(shape, path):
    """Runs that are short or not a multiple of 16 bytes, misaligned
    per-rank bases, a partial sender range (the other windows' blocks keep
    their poison) and a partial receiver range; the automatic kernel choice
    and the LDS kernel forced (small mode-1 unpacks otherwise go direct)."""
    w, B, S, H, D, dtype = shape
    dt = DTYPES[dtype]
    e = torch.empty((), dtype=dt).element_size()
    plan = ua.Plan(w, B, S, H, D, dt)
    plan.set_path(ua.UA2A_PATH_LDS if path == "lds" else ua.UA2A_PATH_AUTO)
    offsets = [(k % 3, (k + 1) % 3, (k + 2) % 3) for k in range(w)] if e < 8 else None
    for mode in (0, 1):
        ish, _ = stacked_shapes(w, B, S, H, D, mode)
        x = make_tensor(ish, dtype, "bytes", 60 + mode)
        senders = list(range(w)) if w < 3 else [0, w - 1]
        receivers = list(range(w)) if w < 3 else list(range(1, w))
        note(f"pack/unpack tail {shape} path {path} mode {mode} senders {senders} receivers {receivers}")
        gw, ww, go, wo = run_pack_unpack(plan, x, mode, senders, receivers, offsets)
        assert_ranks_equal(gw, ww, f"{shape} mode {mode} windows")
        assert_ranks_equal(go, wo, f"{shape} mode {mode} outputs")
    plan.close()
