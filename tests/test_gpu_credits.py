"""GPU tests of readiness credits: the publishing exchange and the wait kernel.

The publishing exchange must give the oracle's bytes and add 1 per call to
every receiving rank's counter.  A consumer on another stream that waits for
a receiver's credit and then copies that receiver's output must see the
oracle's bytes of the CURRENT call (each round uses a new input, so a wait
that returned early would show the previous round's bytes).  A wait whose
target is never reached gives up after its poll limit and reports it.
"""
from __future__ import annotations

import sys

import pytest
import torch

import oracle
import ulysses_all_re_amd as ua
from workloads import BITS_VIEW, CONFIGS, DTYPES, make_tensor

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


def in_shape(w, B, S, H, D, mode):
    return (w, B, S, H, D) if mode == 0 else (w, B, S * w, H // w, D)


@pytest.mark.parametrize("name", ["tiny", "mid", "video_dit", "chunked", "awkward"])
def test_publish_parity_and_counts(name):
    c = CONFIGS[name]
    w, B, S, H, D = c["w"], c["B"], c["S_local"], c["H"], c["D"]
    dt = DTYPES[c["dtype"]]
    plan = ua.Plan(w, B, S, H, D, dt)
    for mode in (0, 1):
        credits = torch.zeros(w, dtype=torch.int32, device=DEV)
        for rnd, parts in ((1, w), (2, 1), (3, max(1, w // 2))):
            x = make_tensor(in_shape(w, B, S, H, D, mode), c["dtype"], "bytes", 100 * mode + rnd)
            note(f"publish {name} mode{mode} round {rnd} parts={parts}")
            out = plan.exchange_publish(x.to(DEV), mode, credits, parts=parts)
            torch.cuda.synchronize()
            assert torch.equal(bits(out.cpu()), oracle_bits(x, mode, w)), (name, mode, rnd)
            assert bool((credits.cpu() == rnd).all()), (name, mode, rnd, credits.tolist())
    plan.close()


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("name", ["video_dit", "chunked"])
def test_consumer_on_another_stream_sees_ready_receivers(name, mode):
    """Stream A runs the publishing exchange (one part per receiver); stream
    B, for each receiving rank in turn, waits for its credit and copies its
    output.  Three rounds with new inputs on the same counters."""
    c = CONFIGS[name]
    w, B, S, H, D = c["w"], c["B"], c["S_local"], c["H"], c["D"]
    dt = DTYPES[c["dtype"]]
    plan = ua.Plan(w, B, S, H, D, dt)
    credits = torch.zeros(w, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.empty(plan.out_shape(mode), dtype=dt, device=DEV)
    snap = torch.empty_like(out)
    side = torch.cuda.Stream(DEV)
    main = torch.cuda.current_stream(DEV)
    for rnd in (1, 2, 3):
        x = make_tensor(in_shape(w, B, S, H, D, mode), c["dtype"], "bytes", 7 * rnd + mode)
        want = oracle_bits(x, mode, w)
        xd = x.to(DEV)
        torch.cuda.synchronize()
        note(f"consumer {name} mode{mode} round {rnd}")
        plan.exchange_publish(xd, mode, credits, out=out, stream=main)
        for r in range(w):
            ua.wait_credits(credits, r, 1, rnd, status, spin_limit=1 << 18, stream=side)
            with torch.cuda.stream(side):
                snap[r].copy_(out[r])
        side.synchronize()
        main.synchronize()
        assert int(status.item()) == 0, (name, mode, rnd)
        assert torch.equal(bits(snap.cpu()), want), (name, mode, rnd)
    plan.close()


def test_wait_gives_up_after_its_poll_limit():
    """Counters that never reach the target: the wait ends by itself after
    spin_limit polls and reports it (the condition is forced from the host)."""
    credits = torch.zeros(64, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    note("wait time-out, spin_limit 1000")
    ua.wait_credits(credits, 0, 64, 1, status, spin_limit=1000)
    torch.cuda.synchronize()
    assert int(status.item()) == 1
    status.zero_()
    credits.fill_(3)
    ua.wait_credits(credits, 0, 64, 3, status, spin_limit=1)     # already reached: no poll needed
    torch.cuda.synchronize()
    assert int(status.item()) == 0


def test_publish_argument_checks():
    plan = ua.Plan(2, 1, 8, 4, 16, torch.bfloat16)
    x = torch.zeros(plan.in_shape(0), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        plan.exchange_publish(x, 0, torch.zeros(1, dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError):
        plan.exchange_publish(x, 0, torch.zeros(2, dtype=torch.int64, device=DEV))
    out = torch.empty(plan.out_shape(0), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ua.UA2AError) as e:
        plan.exchange_publish(x, 0, out.view(torch.int32)[:2], out=out)
    assert e.value.code == ua.UA2A_ERR_ALIAS
    with pytest.raises(ua.UA2AError) as e:
        plan.exchange_publish(x, 0, torch.zeros(2, dtype=torch.int32, device=DEV), parts=3)
    assert e.value.code == ua.UA2A_ERR_INVALID_ARG
    credits = torch.zeros(4, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        ua.wait_credits(credits, 2, 3, 0, torch.zeros(1, dtype=torch.int32, device=DEV))
    plan.close()


def test_publishing_exchange_in_a_hip_graph():
    """Capture a publishing exchange once; every replay (new input copied in,
    eager work and syncs between replays) gives the oracle's bytes and adds
    one more credit per receiver."""
    c = CONFIGS["mid"]
    w, B, S, H, D = c["w"], c["B"], c["S_local"], c["H"], c["D"]
    plan = ua.Plan(w, B, S, H, D, torch.bfloat16)
    credits = torch.zeros(w, dtype=torch.int32, device=DEV)
    x_static = torch.zeros((w, B, S, H, D), dtype=torch.bfloat16, device=DEV)
    y_static = torch.empty(plan.out_shape(0), dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm up outside the capture
        plan.exchange_publish(x_static, 0, credits, out=y_static, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    note("graph capture of a publishing exchange")
    with torch.cuda.graph(graph):
        plan.exchange_publish(x_static, 0, credits, out=y_static)
    for i in range(4):
        x = make_tensor((w, B, S, H, D), "bf16", "bytes", 300 + i)
        x_static.copy_(x.to(DEV))
        bits(y_static).fill_(-1)
        torch.cuda.synchronize()
        note(f"publishing graph replay {i}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(y_static.cpu()), oracle_bits(x, 0, w)), f"replay {i}"
        assert bool((credits.cpu() == i + 2).all()), (i, credits.tolist())
    plan.close()


@pytest.mark.parametrize("blocks", [7, 1000])
def test_publish_with_a_capped_grid(blocks):
    """A `blocks` cap puts the parts on the flat grid-stride kernel, whose
    first workgroup adds the previous part's credits."""
    c = CONFIGS["chunked"]
    w, B, S, H, D = c["w"], c["B"], c["S_local"], c["H"], c["D"]
    plan = ua.Plan(w, B, S, H, D, torch.float16, blocks=blocks)
    for mode in (0, 1):
        credits = torch.zeros(w, dtype=torch.int32, device=DEV)
        x = make_tensor(in_shape(w, B, S, H, D, mode), "fp16", "bytes", 500 + mode)
        note(f"publish blocks={blocks} mode{mode}")
        assert plan.describe(x.to(DEV), mode)["grid_dims"] == 1
        out = plan.exchange_publish(x.to(DEV), mode, credits, parts=w)
        torch.cuda.synchronize()
        assert torch.equal(bits(out.cpu()), oracle_bits(x, mode, w)), (blocks, mode)
        assert bool((credits.cpu() == 1).all()), (blocks, mode, credits.tolist())
    plan.close()


def test_wait_over_more_counters_than_lanes():
    """130 counters: each lane of the wait kernel's wave polls several."""
    credits = torch.full((130,), 5, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    note("wait over 130 counters")
    ua.wait_credits(credits, 0, 130, 5, status, spin_limit=1000)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    credits[129] = 4                              # one short counter, last lane's second pass
    ua.wait_credits(credits, 0, 130, 5, status, spin_limit=1000)
    torch.cuda.synchronize()
    assert int(status.item()) == 1
