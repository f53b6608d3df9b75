"""GPU: the torch operator (forward, backward, torch.compile) and HIP-graph capture.

Forward results, gradients and graph replays are compared with the CPU
oracle bit for bit.  The backward of mode m must equal the oracle's
exchange in mode 1 - m applied to the incoming gradient.
"""
from __future__ import annotations

import sys

import pytest
import torch

import oracle
import ulysses_all_re_amd as ua
from ulysses_all_re_amd import ops
from workloads import BITS_VIEW, CONFIGS, make_tensor

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


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


def oracle_bits(x_cpu, mode, w):
    return torch.from_numpy(oracle.exchange(bits(x_cpu).numpy(), mode, w))


SHAPES = [(2, 1, 8, 4, 16), (4, 2, 100, 8, 64), (3, 2, 33, 12, 80)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forward_matches_oracle(shape):
    w, B, S, H, D = shape
    x = make_tensor(shape, "bf16", "normal", 3)
    note(f"ops forward {shape}")
    y = ops.all_to_all_4D(x.to(DEV), 2, 1, w)
    assert torch.equal(bits(y.cpu()), oracle_bits(x, 0, w))
    z = ops.all_to_all_4D(y, 1, 2, w)
    assert torch.equal(bits(z.cpu()), bits(x))


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_is_the_inverse_exchange(shape):
    w, B, S, H, D = shape
    x = make_tensor(shape, "fp32", "normal", 4).to(DEV).requires_grad_(True)
    note(f"ops backward {shape}")
    y = ops.all_to_all_4D(x, 2, 1, w)
    g = make_tensor(tuple(y.shape), "fp32", "normal", 5)
    y.backward(g.to(DEV))
    assert torch.equal(bits(x.grad.cpu()), oracle_bits(g, 1, w))
    # and through mode 1 as the forward
    u = make_tensor(tuple(y.shape), "fp32", "normal", 6).to(DEV).requires_grad_(True)
    v = ops.all_to_all_4D(u, 1, 2, w)
    h = make_tensor(tuple(v.shape), "fp32", "normal", 7)
    v.backward(h.to(DEV))
    assert torch.equal(bits(u.grad.cpu()), oracle_bits(h, 0, w))


def test_chunked_operator_grows_its_window():
    """chunked=True: one window per device and stream, grown when a larger shape
    arrives (the plans that borrowed the old one are rebuilt) and never shrunk;
    every result, forward and backward, equals the unchunked one and the oracle."""
    side = torch.cuda.Stream()
    shapes = [(2, 2, 8, 4, 16), (4, 3, 100, 8, 64), (2, 2, 8, 4, 16), (3, 2, 33, 12, 80)]
    sizes = []
    with torch.cuda.stream(side):
        for k, (w, B, S, H, D) in enumerate(shapes):
            x = make_tensor((w, B, S, H, D), "bf16", "bytes", 70 + k)
            xd = x.to(DEV).requires_grad_(False)
            note(f"chunked op {(w, B, S, H, D)}")
            y = ops.all_to_all_4D(xd, 2, 1, w, chunked=True)
            z = ops.all_to_all_4D(y, 1, 2, w, chunked=True)
            side.synchronize()
            assert torch.equal(bits(y.cpu()), oracle_bits(x, 0, w)), k
            assert torch.equal(bits(z.cpu()), bits(x)), k
            sizes.append(ops._windows[(torch.device(DEV), side.stream_id)].numel())
    e = 2
    need = [w * S * H * D * e for (w, B, S, H, D) in shapes]
    assert sizes == [max(need[:i + 1]) for i in range(len(shapes))]     # grows, never shrinks
    # a chunked plan borrows the current window; the one built on the first window is gone
    win = ops._windows[(torch.device(DEV), side.stream_id)]
    chunked_plans = [p for key, p in ops._plans.items() if len(key) == 8 and key[-1] == side.stream_id]
    assert chunked_plans and all(p.window is win for p in chunked_plans)
    # backward of a chunked mode 0 is the chunked mode 1
    w, B, S, H, D = 3, 2, 33, 12, 80
    x = make_tensor((w, B, S, H, D), "fp32", "normal", 79).to(DEV).requires_grad_(True)
    y = ops.all_to_all_4D(x, 2, 1, w, chunked=True)
    g = make_tensor(tuple(y.shape), "fp32", "normal", 80)
    y.backward(g.to(DEV))
    assert torch.equal(bits(x.grad.cpu()), oracle_bits(g, 1, w))


def test_chunked_operator_caches_are_bounded_and_growth_is_logged(monkeypatch, caplog):
    """Chunked calls on more streams than MAX_WINDOWS keep at most that many
    windows (and at most MAX_PLANS plans); each window's creation and growth
    is logged; every result matches the oracle."""
    monkeypatch.setattr(ops, "MAX_WINDOWS", 2)
    monkeypatch.setattr(ops, "MAX_PLANS", 3)
    streams = [torch.cuda.Stream() for _ in range(4)]
    shapes = [(2, 2, 8, 4, 16), (2, 2, 16, 4, 16)]          # the second needs a larger window
    caplog.set_level("INFO", logger=ops.__name__)
    for k, st in enumerate(streams):
        with torch.cuda.stream(st):
            for j, (w, B, S, H, D) in enumerate(shapes):
                x = make_tensor((w, B, S, H, D), "bf16", "bytes", 90 + 2 * k + j)
                note(f"bounded caches stream {k} shape {(w, B, S, H, D)}")
                y = ops.all_to_all_4D(x.to(DEV), 2, 1, w, chunked=True)
                st.synchronize()
                assert torch.equal(bits(y.cpu()), oracle_bits(x, 0, w)), (k, j)
        assert len(ops._windows) <= 2 and len(ops._plans) <= 3
    grown = [r for r in caplog.records if "grown from" in r.getMessage()]
    created = [r for r in caplog.records if "created with" in r.getMessage()]
    assert len(grown) >= len(streams) and len(created) >= len(streams)


def test_torch_compile_traces_the_operator():
    w, B, S, H, D = 4, 2, 64, 8, 32
    x = make_tensor((w, B, S, H, D), "fp16", "uniform", 8).to(DEV)

    def block(t):
        y = ops.all_to_all_4D(t, 2, 1, w)           # heads -> sequence
        y = y * 2                                     # stand-in for attention
        return ops.all_to_all_4D(y, 1, 2, w)          # back

    note("torch.compile aot_eager fullgraph")
    compiled = torch.compile(block, backend="aot_eager", fullgraph=True)
    got = compiled(x)
    torch.cuda.synchronize()
    assert torch.equal(got, block(x))
    assert torch.equal(got, x * 2)


# ------------------------------------------------------------- graph capture

@pytest.mark.parametrize("chunked", [False, True])
def test_hip_graph_capture_and_replay(chunked):
    """Capture an exchange (and its inverse) once; replay with new inputs copied in
    between replays, eager work and syncs interleaved; every replay must match."""
    c = CONFIGS["chunked"]
    w, B, S, H, D = c["w"], c["B"], c["S_local"], c["H"], c["D"]
    lay = ua.ua2a_layout(w, B, S, H, D, 2)
    window = torch.empty(lay["window_bytes"], dtype=torch.uint8, device=DEV)
    plan = ua.Plan(w, B, S, H, D, torch.float16, window=window)
    x_static = torch.zeros((w, B, S, H, D), dtype=torch.float16, device=DEV)
    y_static = torch.empty(plan.out_shape(0), dtype=torch.float16, device=DEV)
    z_static = torch.empty(plan.out_shape(1), dtype=torch.float16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm up outside the capture
        plan.exchange(x_static, 0, chunked, out=y_static)
        plan.exchange(y_static, 1, chunked, out=z_static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    note(f"graph capture chunked={chunked}")
    with torch.cuda.graph(graph):
        plan.exchange(x_static, 0, chunked, out=y_static)
        plan.exchange(y_static, 1, chunked, out=z_static)
    y_addr = y_static.data_ptr()
    for i in range(4):
        x = make_tensor((w, B, S, H, D), "fp16", "uniform", 100 + i)
        x_static.copy_(x.to(DEV))
        bits(y_static).fill_(-1)                  # eager work between replays
        bits(z_static).fill_(-1)
        torch.cuda.synchronize()
        note(f"graph replay {i} chunked={chunked}")
        graph.replay()
        torch.cuda.synchronize()
        assert y_static.data_ptr() == y_addr
        assert torch.equal(bits(y_static.cpu()), oracle_bits(x, 0, w)), f"replay {i}"
        assert torch.equal(bits(z_static.cpu()), bits(x)), f"replay {i}"
    plan.close()
