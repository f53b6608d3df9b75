"""GPU parity: the HIP exchange, called through the C ABI, against the CPU oracle.

Every comparison is byte for byte (the exchange is a pure permutation, so the
bar is bit-exactness for every dtype).  Covers the five workloads at their
full sizes, both modes, the chunked path, the short-run and unaligned tail
paths, both kernel families, misaligned bases, grid-size hints, poisoned
outputs and guard bands, back-to-back launches on one stream, a non-default
stream, and the argument checks.
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
POISON = -1          # 0xFF.. bit pattern written into outputs before each run
PATHS = {"auto": ua.UA2A_PATH_AUTO, "direct": ua.UA2A_PATH_DIRECT, "lds": ua.UA2A_PATH_LDS}


def note(msg):
    """Name the case on stdout before it touches the GPU."""
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


def oracle_out(x_cpu, mode, w, chunked=False):
    xb = bits(x_cpu).numpy()
    return torch.from_numpy(oracle.exchange(xb, mode, w, chunked=chunked))


def poisoned(shape, dtype):
    t = torch.empty(shape, dtype=dtype, device=DEV)
    b = bits(t)
    b.fill_(255 if b.dtype == torch.uint8 else POISON)     # all-ones bit pattern
    return t


def assert_same_bits(got_dev, want_bits_cpu, what):
    got = bits(got_dev.cpu())
    if not torch.equal(got, want_bits_cpu):
        bad = (got != want_bits_cpu).nonzero()
        raise AssertionError(f"{what}: {bad.shape[0]} elements differ; first at {bad[0].tolist()}")


def cfg_shape(c):
    return c["w"], c["B"], c["S_local"], c["H"], c["D"]


def in_shape(w, B, S, H, D, mode):
    return (w, B, S, H, D) if mode == 0 else (w, B, S * w, H // w, D)


# ------------------------------------------------------------ the workloads

@pytest.mark.parametrize("name", ["tiny", "mid", "video_dit", "chunked", "awkward"])
def test_workload_parity(name):
    c = CONFIGS[name]
    w, B, S, H, D = cfg_shape(c)
    dt = ua_dtype = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[c["dtype"]]
    lay = ua.ua2a_layout(w, B, S, H, D, torch.empty((), dtype=dt).element_size())
    window = torch.empty(lay["window_bytes"], dtype=torch.uint8, device=DEV) if c["chunked"] else None
    plan = ua.Plan(w, B, S, H, D, ua_dtype, window=window)
    chunk_opts = (False, True) if c["chunked"] else (False,)
    x0 = make_tensor(in_shape(w, B, S, H, D, 0), c["dtype"], c["dist"], c["seed0"])
    want0 = oracle_out(x0, 0, w)
    x0d = x0.to(DEV)
    for chunked in chunk_opts:
        note(f"{name} mode0 chunked={chunked} shape={tuple(x0.shape)} path={plan.describe(x0d, 0, chunked)}")
        y = plan.exchange(x0d, 0, chunked, out=poisoned(plan.out_shape(0), dt))
        torch.cuda.synchronize()
        assert_same_bits(y, want0, f"{name} mode 0 chunked={chunked}")
        # round trip: mode 1 on mode 0's output gives the input back
        note(f"{name} mode1 round trip chunked={chunked}")
        z = plan.exchange(y, 1, chunked, out=poisoned(plan.out_shape(1), dt))
        torch.cuda.synchronize()
        assert_same_bits(z, bits(x0), f"{name} round trip chunked={chunked}")
    del want0, y, z
    # mode 1 on an independent input
    dist = c["dist"] if c["dist"] != "index" else "index_bits"
    x1 = make_tensor(in_shape(w, B, S, H, D, 1), c["dtype"], dist, c["seed1"])
    want1 = oracle_out(x1, 1, w)
    x1d = x1.to(DEV)
    for chunked in chunk_opts:
        note(f"{name} mode1 chunked={chunked} shape={tuple(x1.shape)}")
        u = plan.exchange(x1d, 1, chunked, out=poisoned(plan.out_shape(1), dt))
        torch.cuda.synchronize()
        assert_same_bits(u, want1, f"{name} mode 1 chunked={chunked}")
    plan.close()


def test_awkward_exact_provenance():
    """The awkward workload with every element a distinct int32 bit pattern."""
    c = CONFIGS["awkward"]
    w, B, S, H, D = cfg_shape(c)
    x = make_tensor((w, B, S, H, D), "fp32", "index_bits")
    plan = ua.Plan(w, B, S, H, D, torch.float32)
    note("awkward index_bits mode0")
    y = plan.exchange(x.to(DEV), 0).cpu()
    got = bits(y).numpy()
    # decode where each element came from and check it against the oracle's placement
    assert np.array_equal(got, oracle.exchange(bits(x).numpy(), 0, w))
    assert np.array_equal(np.sort(got.ravel()), np.arange(x.numel(), dtype=np.int32))
    plan.close()


# ------------------------------------------------- tail shapes, both paths

@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("shape", TAIL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_tail_shapes(shape, path):
    w, B, S, H, D, dtype = shape
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32,
          "f64": torch.float64, "u8": torch.uint8}[dtype]
    e = torch.empty((), dtype=dt).element_size()
    lay = ua.ua2a_layout(w, B, S, H, D, e)
    window = torch.empty(lay["window_bytes"], dtype=torch.uint8, device=DEV)
    plan = ua.Plan(w, B, S, H, D, dt, window=window)
    plan.set_path(PATHS[path])
    for mode in (0, 1):
        x = make_tensor(in_shape(w, B, S, H, D, mode), dtype, "bytes", 11 + mode)
        want = oracle_out(x, mode, w)
        xd = x.to(DEV)
        for chunked in (False, True):
            note(f"tail {shape} {path} mode={mode} chunked={chunked} {plan.describe(xd, mode, chunked)}")
            y = plan.exchange(xd, mode, chunked, out=poisoned(plan.out_shape(mode), dt))
            torch.cuda.synchronize()
            assert_same_bits(y, want, f"tail {shape} {path} mode {mode} chunked={chunked}")
    plan.close()


@pytest.mark.parametrize("offsets", [(1, 0), (0, 1), (1, 3), (5, 7)])
@pytest.mark.parametrize("shape", [(4, 1, 1024, 24, 128, "bf16"), (3, 1, 5, 3, 7, "bf16"),
                                   (2, 2, 300, 4, 16, "bf16")], ids=lambda s: "x".join(map(str, s)))
def test_misaligned_bases(shape, offsets):
    """Tensors that start one or more elements past an aligned address, with guard bands."""
    w, B, S, H, D, dtype = shape
    dt = torch.bfloat16
    plan = ua.Plan(w, B, S, H, D, dt)
    n = w * B * S * H * D
    for path in ("auto", "direct", "lds"):
        plan.set_path(PATHS[path])
        for mode in (0, 1):
            x = make_tensor(in_shape(w, B, S, H, D, mode), dtype, "normal", 21 + mode)
            want = oracle_out(x, mode, w)
            xin = torch.zeros(n + 64, dtype=dt, device=DEV)
            xin[offsets[0]:offsets[0] + n] = x.reshape(-1).to(DEV)
            outbuf = poisoned((n + 64,), dt)
            xi = xin[offsets[0]:offsets[0] + n].view(in_shape(w, B, S, H, D, mode))
            yo = outbuf[offsets[1]:offsets[1] + n].view(plan.out_shape(mode))
            note(f"misaligned {shape} {offsets} {path} mode={mode} {plan.describe(xi, mode, out=yo)}")
            plan.exchange(xi, mode, out=yo)
            torch.cuda.synchronize()
            assert_same_bits(yo, want, f"misaligned {shape} {offsets} {path} mode {mode}")
            guard = bits(outbuf.cpu())
            assert (guard[:offsets[1]] == POISON).all() and (guard[offsets[1] + n:] == POISON).all()
    plan.close()


@pytest.mark.parametrize("shape", [(8, 1, 2048, 8, 256), (4, 2, 513, 8, 512), (2, 3, 37, 2, 1024)],
                         ids=lambda s: "x".join(map(str, s)))
def test_power_of_two_rows(shape):
    """Token rows that are a multiple of 4 KiB take the interleaved tile order in mode 0."""
    w, B, S, H, D = shape
    plan = ua.Plan(w, B, S, H, D, torch.bfloat16)
    for mode in (0, 1):
        x = make_tensor(in_shape(w, B, S, H, D, mode), "bf16", "normal", 31 + mode)
        want = oracle_out(x, mode, w)
        xd = x.to(DEV)
        note(f"pow2 rows {shape} mode={mode} {plan.describe(xd, mode)}")
        y = plan.exchange(xd, mode, out=poisoned(plan.out_shape(mode), torch.bfloat16))
        torch.cuda.synchronize()
        assert_same_bits(y, want, f"pow2 rows {shape} mode {mode}")
    plan.close()


@pytest.mark.parametrize("S", [20479, 20480], ids=["under-80MiB", "at-80MiB"])
def test_mode1_kernel_choice_at_its_size_boundary(S):
    """Mode 1 on 64-byte runs takes the direct kernel just under 80 MiB a side
    and the LDS kernel at 80 MiB; either way the output equals the oracle's and
    mode 0 on it returns the input."""
    w, B, H, D = 8, 1, 8, 32
    plan = ua.Plan(w, B, S, H, D, torch.bfloat16)
    x = make_tensor(in_shape(w, B, S, H, D, 1), "bf16", "bytes", 880 + S % 2)
    want = oracle_out(x, 1, w)
    xd = x.to(DEV)
    info = plan.describe(xd, 1, False)
    assert info["path"] == (ua.UA2A_PATH_DIRECT if S < 20480 else ua.UA2A_PATH_LDS), info
    note(f"mode 1 size boundary S={S} path={info['path']}")
    y = plan.exchange(xd, 1, out=poisoned(plan.out_shape(1), torch.bfloat16))
    torch.cuda.synchronize()
    assert_same_bits(y, want, f"mode 1 S={S}")
    note(f"mode 0 round trip S={S}")
    z = plan.exchange(y, 0, out=poisoned(plan.out_shape(0), torch.bfloat16))
    torch.cuda.synchronize()
    assert_same_bits(z, bits(x), f"round trip S={S}")
    plan.close()


def test_large_tensor_sampled():
    """16 GiB per tensor (2^31 eight-byte elements): byte offsets far past 2^32.
    Each element holds its own input position, so a sampled output position
    must hold exactly what the element oracle says it came from."""
    w, B, S, H, D = 8, 2, 32768, 64, 64
    n = w * B * S * H * D
    assert n == 2 ** 31
    lay = ua.ua2a_layout(w, B, S, H, D, 8)
    window = torch.empty(lay["window_bytes"], dtype=torch.uint8, device=DEV)
    plan = ua.Plan(w, B, S, H, D, torch.int64, window=window)
    x = torch.arange(n, dtype=torch.int64, device=DEV).view(w, B, S, H, D)
    gen = torch.Generator("cpu").manual_seed(12)
    idx = torch.cat([torch.arange(4096), torch.randint(0, n, (200000,), generator=gen),
                     torch.arange(n - 4096, n)])
    for mode in (0, 1):
        for chunked in (False, True):
            note(f"large sampled mode={mode} chunked={chunked} {plan.describe(x, mode, chunked)}")
            src = x if mode == 0 else x.view(plan.in_shape(1))
            y = plan.exchange(src, mode, chunked)
            torch.cuda.synchronize()
            got = y.view(-1)[idx.to(DEV)].cpu().numpy()
            want = oracle.source_indices(mode, w, B, S, H, D, idx.numpy())
            assert np.array_equal(got, want), (mode, chunked)
            del y
    note("large round trip")
    y = plan.exchange(x, 0)
    z = plan.exchange(y, 1)
    torch.cuda.synchronize()
    assert torch.equal(z, x)
    plan.close()


@pytest.mark.parametrize("B", [1, 3], ids=["2GiB", "6GiB"])
def test_lds_path_sampled_around_4_gib(B):
    """32-byte runs (the LDS path, 16-byte pieces) on rank-stacked tensors of 2 GiB
    (mode 0 stores each tile's spans through one range) and 6 GiB (too large for
    one range: plain stores): sampled outputs against the element oracle, both
    modes, chunked and not, and a full round trip."""
    w, S, H, D = 8, 2 ** 20, 8, 4
    n = w * B * S * H * D
    lay = ua.ua2a_layout(w, B, S, H, D, 8)
    window = torch.empty(lay["window_bytes"], dtype=torch.uint8, device=DEV)
    plan = ua.Plan(w, B, S, H, D, torch.int64, window=window)
    plan.set_path(ua.UA2A_PATH_LDS)
    x = torch.arange(n, dtype=torch.int64, device=DEV).view(w, B, S, H, D)
    gen = torch.Generator("cpu").manual_seed(13 + B)
    idx = torch.cat([torch.arange(4096), torch.randint(0, n, (200000,), generator=gen),
                     torch.arange(n - 4096, n)])
    for mode in (0, 1):
        for chunked in (False, True):
            info = plan.describe(x, mode, chunked)
            assert info["path"] == ua.UA2A_PATH_LDS and info["vector_bytes"] == 16
            note(f"LDS sampled B={B} mode={mode} chunked={chunked} {info}")
            src = x if mode == 0 else x.view(plan.in_shape(1))
            y = plan.exchange(src, mode, chunked)
            torch.cuda.synchronize()
            got = y.view(-1)[idx.to(DEV)].cpu().numpy()
            want = oracle.source_indices(mode, w, B, S, H, D, idx.numpy())
            assert np.array_equal(got, want), (mode, chunked)
            del y
    note(f"LDS round trip B={B}")
    y = plan.exchange(x, 0)
    z = plan.exchange(y, 1)
    torch.cuda.synchronize()
    assert torch.equal(z, x)
    plan.close()


def test_capped_grid_at_64_gib():
    """64 GiB per tensor with 4 KiB token rows: mode 0 runs the flat grouped
    order with 2^26 tiles, more than one dispatch can count in lanes, so the
    grid is capped and every workgroup loops over several tiles."""
    w, B, S, H, D = 8, 16, 2 ** 17, 8, 64          # 8-byte elements, 512-byte runs
    n = w * B * S * H * D
    free, _ = torch.cuda.mem_get_info()
    if free < 140 * 2 ** 30:
        pytest.skip(f"needs about 130 GiB of free device memory, {free / 2 ** 30:.0f} GiB free")
    torch.cuda.empty_cache()
    plan = ua.Plan(w, B, S, H, D, torch.int64)
    x = torch.empty(n, dtype=torch.int64, device=DEV)
    step = 2 ** 27                                 # torch's own fill kernels stay small
    for a in range(0, n, step):
        x[a:a + step] = torch.arange(a, min(n, a + step), dtype=torch.int64, device=DEV)
    x = x.view(w, B, S, H, D)
    info = plan.describe(x, 0)
    assert info["grid_dims"] == 1 and info["grid"] * info["block"] <= 2 ** 31 < info["tiles"] * 64
    note(f"64 GiB mode 0 {info}")
    y = plan.exchange(x, 0)
    torch.cuda.synchronize()
    gen = torch.Generator("cpu").manual_seed(64)
    idx = torch.cat([torch.arange(4096), torch.randint(0, n, (200000,), generator=gen),
                     torch.arange(n - 4096, n)])
    got = y.view(-1)[idx.to(DEV)].cpu().numpy()
    assert np.array_equal(got, oracle.source_indices(0, w, B, S, H, D, idx.numpy()))
    del x
    note("64 GiB mode 1 round trip")
    z = plan.exchange(y, 1)
    torch.cuda.synchronize()
    del y
    for a in range(0, n, step):
        b = min(n, a + step)
        assert torch.equal(z.view(-1)[a:b], torch.arange(a, b, dtype=torch.int64, device=DEV)), a
    del z
    plan.close()
    torch.cuda.empty_cache()


def _random_cases(n, seed):
    """Seeded random shapes, element sizes, paths, modes and misalignments."""
    rng = np.random.default_rng(seed)
    dts = [("u8", torch.uint8), ("bf16", torch.bfloat16), ("fp32", torch.float32),
           ("f64", torch.float64)]
    cases = []
    for _ in range(n):
        w = int(rng.integers(1, 9))
        hl = int(rng.integers(1, 7))
        name, dt = dts[int(rng.integers(0, len(dts)))]
        e = torch.empty((), dtype=dt).element_size()
        B, S, D = int(rng.integers(1, 4)), int(rng.integers(1, 700)), int(rng.integers(1, 200))
        S = max(1, min(S, (32 << 20) // (w * B * w * hl * D * e)))    # at most ~32 MB per tensor
        cases.append(dict(w=w, B=B, S=S, H=w * hl, D=D, name=name, dt=dt, e=e,
                          mode=int(rng.integers(0, 2)), chunked=bool(rng.integers(0, 2)),
                          path=["auto", "direct", "lds"][int(rng.integers(0, 3))],
                          mis_in=int(rng.integers(0, 4)), mis_out=int(rng.integers(0, 4))))
    return cases


@pytest.mark.parametrize("case", _random_cases(60, 2024), ids=lambda c: (
    f"w{c['w']}B{c['B']}S{c['S']}H{c['H']}D{c['D']}{c['name']}m{c['mode']}"
    f"{'c' if c['chunked'] else ''}{c['path']}{c['mis_in']}{c['mis_out']}"))
def test_random_cases(case):
    w, B, S, H, D, dt = case["w"], case["B"], case["S"], case["H"], case["D"], case["dt"]
    n = w * B * S * H * D
    mode = case["mode"]
    lay = ua.ua2a_layout(w, B, S, H, D, case["e"])
    window = torch.empty(lay["window_bytes"] + 64, dtype=torch.uint8, device=DEV)
    plan = ua.Plan(w, B, S, H, D, dt, window=window)
    plan.set_path(PATHS[case["path"]])
    x = make_tensor(in_shape(w, B, S, H, D, mode), case["name"], "bytes", n % 9973)
    want = oracle_out(x, mode, w)
    xin = torch.zeros(n + 8, dtype=dt, device=DEV)
    xin[case["mis_in"]:case["mis_in"] + n] = x.reshape(-1).to(DEV)
    outbuf = poisoned((n + 8,), dt)
    xi = xin[case["mis_in"]:case["mis_in"] + n].view(in_shape(w, B, S, H, D, mode))
    yo = outbuf[case["mis_out"]:case["mis_out"] + n].view(plan.out_shape(mode))
    note(f"random {case} {plan.describe(xi, mode, case['chunked'], out=yo)}")
    plan.exchange(xi, mode, case["chunked"], out=yo)
    torch.cuda.synchronize()
    assert_same_bits(yo, want, f"random case {case}")
    guard = bits(outbuf.cpu())
    full = 255 if guard.dtype == torch.uint8 else POISON
    assert (guard[:case["mis_out"]] == full).all() and (guard[case["mis_out"] + n:] == full).all()
    plan.close()


def _random_chunked_cases(n, seed):
    """Seeded chunked exchanges of 2-9 planes on the direct path (one launch of
    the chunked kernel), misaligned bases included."""
    rng = np.random.default_rng(seed)
    cases = []
    for c in _random_cases(n, seed):
        c.update(B=int(rng.integers(2, 10)), chunked=True, path="direct")
        c["S"] = max(1, min(c["S"], (32 << 20) // (c["w"] * c["B"] * c["H"] * c["D"] * c["e"])))
        cases.append(c)
    return cases


@pytest.mark.parametrize("case", _random_chunked_cases(24, 4242), ids=lambda c: (
    f"w{c['w']}B{c['B']}S{c['S']}H{c['H']}D{c['D']}{c['name']}m{c['mode']}{c['mis_in']}{c['mis_out']}"))
def test_random_chunked_one_launch(case):
    w, B, S, H, D, dt = case["w"], case["B"], case["S"], case["H"], case["D"], case["dt"]
    n = w * B * S * H * D
    mode = case["mode"]
    lay = ua.ua2a_layout(w, B, S, H, D, case["e"])
    window = torch.full((lay["window_bytes"] + 256,), 0x3C, dtype=torch.uint8, device=DEV)
    plan = ua.Plan(w, B, S, H, D, dt, window=window[:lay["window_bytes"]])
    plan.set_path(ua.UA2A_PATH_DIRECT)
    x = make_tensor(in_shape(w, B, S, H, D, mode), case["name"], "bytes", n % 7919)
    want = oracle_out(x, mode, w)
    xin = torch.zeros(n + 8, dtype=dt, device=DEV)
    xin[case["mis_in"]:case["mis_in"] + n] = x.reshape(-1).to(DEV)
    outbuf = poisoned((n + 8,), dt)
    xi = xin[case["mis_in"]:case["mis_in"] + n].view(in_shape(w, B, S, H, D, mode))
    yo = outbuf[case["mis_out"]:case["mis_out"] + n].view(plan.out_shape(mode))
    info = plan.describe(xi, mode, True, out=yo)
    note(f"random chunked {case} {info}")
    plan.exchange(xi, mode, True, out=yo)
    torch.cuda.synchronize()
    assert_same_bits(yo, want, f"random chunked case {case}")
    guard = bits(outbuf.cpu())
    full = 255 if guard.dtype == torch.uint8 else POISON
    assert (guard[:case["mis_out"]] == full).all() and (guard[case["mis_out"] + n:] == full).all()
    assert (window[lay["window_bytes"]:].cpu() == 0x3C).all()
    last = want.view(torch.uint8).reshape(w, B, -1)[:, B - 1]
    assert torch.equal(window[:lay["window_bytes"]].cpu().reshape(w, -1), last), f"window after {case}"
    if info["grid_dims"] == 3:
        assert info["launches"] == 1 and info["chunked_form"] == ua.UA2A_CHUNKED_ONE_LAUNCH
    plan.close()


# ------------------------------------------------------ launch-shape freedom

@pytest.mark.parametrize("blocks", [1, 7, 64, 0])
def test_blocks_hint_gives_identical_bytes(blocks):
    w, B, S, H, D = cfg_shape(CONFIGS["mid"])
    x = make_tensor((w, B, S, H, D), "bf16", "normal", 0)
    want = oracle_out(x, 0, w)
    xd = x.to(DEV)
    for path in ("direct", "lds"):
        plan = ua.Plan(w, B, S, H, D, torch.bfloat16, blocks=blocks)
        plan.set_path(PATHS[path])
        note(f"blocks={blocks} path={path} {plan.describe(xd, 0)}")
        y = plan.exchange(xd, 0, out=poisoned(plan.out_shape(0), torch.bfloat16))
        torch.cuda.synchronize()
        assert_same_bits(y, want, f"blocks={blocks} {path}")
        z = plan.exchange(y, 1)
        torch.cuda.synchronize()
        assert_same_bits(z, bits(x), f"blocks={blocks} {path} round trip")
        plan.close()


@pytest.mark.parametrize("blocks", [1, 7, 300, 5000])
@pytest.mark.parametrize("shape", [(4, 4, 2048, 16, 64, "fp16"), (2, 3, 37, 2, 1024, "bf16"),
                                   (3, 2, 41, 3, 5, "fp32")], ids=lambda s: "x".join(map(str, s)))
def test_chunked_under_a_blocks_hint(shape, blocks):
    """A chunked exchange on a grid capped by a blocks hint stays one launch: on the
    direct path the chunked kernel's flat form, each workgroup moving several window
    tiles in turn (4 KiB rows: in the grouped tile order, padding tiles included); on
    the LDS path the chunked LDS kernel's slot loop.  Bytes and window as without it."""
    w, B, S, H, D, dtype = shape
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]
    e = torch.empty((), dtype=dt).element_size()
    lay = ua.ua2a_layout(w, B, S, H, D, e)
    win = torch.empty(lay["window_bytes"], dtype=torch.uint8, device=DEV)
    plan = ua.Plan(w, B, S, H, D, dt, blocks=blocks, window=win)
    for path in ("direct", "lds"):
        plan.set_path(PATHS[path])
        for mode in (0, 1):
            x = make_tensor(in_shape(w, B, S, H, D, mode), dtype, "bytes", 80 + mode)
            want = oracle_out(x, mode, w)
            xd = x.to(DEV)
            info = plan.describe(xd, mode, True)
            assert info["launches"] == 1 and info["grid"] <= blocks
            note(f"chunked blocks={blocks} {shape} {path} mode={mode} {info}")
            y = plan.exchange(xd, mode, True, out=poisoned(plan.out_shape(mode), dt))
            torch.cuda.synchronize()
            assert_same_bits(y, want, f"chunked blocks={blocks} {shape} {path} mode {mode}")
            last = want.view(torch.uint8).reshape(w, B, -1)[:, B - 1]
            assert torch.equal(win.cpu().reshape(w, -1), last), f"window {shape} {path} {mode}"
    plan.close()


def test_back_to_back_on_one_stream_and_side_stream():
    """mode 0 -> mode 1 -> mode 0 queued without host syncs, on a non-default stream."""
    w, B, S, H, D = cfg_shape(CONFIGS["chunked"])
    x = make_tensor((w, B, S, H, D), "fp16", "uniform", 0)
    want = oracle_out(x, 0, w)
    lay = ua.ua2a_layout(w, B, S, H, D, 2)
    window = torch.empty(lay["window_bytes"], dtype=torch.uint8, device=DEV)
    plan = ua.Plan(w, B, S, H, D, torch.float16, window=window)
    s = torch.cuda.Stream()
    xd = x.to(DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        note("back-to-back chunked/unchunked on a side stream")
        y = plan.exchange(xd, 0, True)
        z = plan.exchange(y, 1, False)
        y2 = plan.exchange(z, 0, False)
        z2 = plan.exchange(y2, 1, True)
    s.synchronize()
    assert_same_bits(y, want, "chunked mode 0")
    assert_same_bits(y2, want, "mode 0 after round trip")
    assert_same_bits(z2, bits(x), "second round trip")
    plan.close()


@pytest.mark.parametrize("shape", [(4, 1, 60001, 4, 7), (130, 1, 37, 130, 7), (8, 2, 1001, 8, 3)],
                         ids=lambda s: "x".join(map(str, s)))
def test_lds_spans_misaligned_to_16_bytes(shape):
    """Odd S_local with runs that are not a multiple of 16 B: the LDS path's A spans
    start and end inside 16-byte chunks, which mode 1 reads whole (w = 130: more
    such chunks per tile than lanes).  Stacked and, for w <= 64, per-rank calls,
    both modes, against the oracle."""
    w, B, S, H, D = shape
    plan = ua.Plan(w, B, S, H, D, torch.bfloat16)
    plan.set_path(ua.UA2A_PATH_LDS)
    for mode in (0, 1):
        x = make_tensor(in_shape(w, B, S, H, D, mode), "bf16", "bytes", 60 + mode)
        want = oracle_out(x, mode, w)
        xd = x.to(DEV)
        out = poisoned(plan.out_shape(mode), torch.bfloat16)
        info = plan.describe(xd, mode, out=out)
        assert info["path"] == ua.UA2A_PATH_LDS and info["vector_bytes"] < 16
        note(f"misaligned LDS spans {shape} mode {mode}")
        plan.exchange(xd, mode, out=out)
        torch.cuda.synchronize()
        assert_same_bits(out, want, f"stacked mode {mode}")
        if w <= ua.MAX_RANK_TABLE:
            xs = [xd[k].clone() for k in range(w)]
            outs = [poisoned(plan.out_shape(mode)[1:], torch.bfloat16) for _ in range(w)]
            assert plan.describe_ranks(xs, outs, mode)["path"] == ua.UA2A_PATH_LDS
            plan.exchange_ranks(xs, mode, outs=outs)
            torch.cuda.synchronize()
            assert_same_bits(torch.stack(outs), want, f"per-rank mode {mode}")
    plan.close()


def test_independent_plans_on_concurrent_streams():
    """Four plans, two of them chunked with windows of their own, each running
    three round trips on its own stream with no host sync in between: the
    plans share no device state, so every stream ends with the oracle's bytes."""
    cases = [((4, 1, 1024, 24, 128), "bf16", False), ((3, 2, 33, 12, 80), "fp32", True),
             ((2, 3, 37, 2, 1024), "bf16", True), ((8, 1, 13, 40, 128), "fp16", False)]
    dts = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
    jobs = []
    for k, ((w, B, S, H, D), dt, chunked) in enumerate(cases):
        x = make_tensor((w, B, S, H, D), dt, "bytes", 40 + k)
        e = x.element_size()
        lay = ua.ua2a_layout(w, B, S, H, D, e)
        window = torch.empty(lay["window_bytes"], dtype=torch.uint8, device=DEV) if chunked else None
        plan = ua.Plan(w, B, S, H, D, dts[dt], window=window)
        y = poisoned(plan.out_shape(0), dts[dt])
        z = poisoned(plan.in_shape(0), dts[dt])
        jobs.append((plan, x, x.to(DEV), y, z, chunked, torch.cuda.Stream(), oracle_out(x, 0, w)))
    torch.cuda.synchronize()
    note("4 plans on 4 concurrent streams, 3 round trips each")
    for _ in range(3):
        for plan, _, xd, y, z, chunked, st, _ in jobs:
            with torch.cuda.stream(st):
                plan.exchange(xd, 0, chunked, out=y)
                plan.exchange(y, 1, chunked, out=z)
    torch.cuda.synchronize()
    for k, (plan, x, _, y, z, chunked, _, want) in enumerate(jobs):
        assert_same_bits(y, want, f"stream {k} mode 0")
        assert_same_bits(z, bits(x), f"stream {k} round trip")
        plan.close()


def test_window_is_reused_and_left_alone_outside_its_size():
    """Chunked planes share one window; bytes past the one-plane size stay untouched."""
    w, B, S, H, D = 4, 3, 100, 8, 32
    lay = ua.ua2a_layout(w, B, S, H, D, 2)
    win = torch.full((lay["window_bytes"] + 4096,), 0x77, dtype=torch.uint8, device=DEV)
    plan = ua.Plan(w, B, S, H, D, torch.bfloat16, window=win)
    x = make_tensor((w, B, S, H, D), "bf16", "normal", 4)
    note("window reuse")
    y = plan.exchange(x.to(DEV), 0, True)
    torch.cuda.synchronize()
    assert_same_bits(y, oracle_out(x, 0, w), "chunked via shared window")
    assert (win[lay["window_bytes"]:].cpu() == 0x77).all()
    plan.close()


@pytest.mark.parametrize("shape", [(4, 5, 96, 8, 64, "bf16"), (3, 2, 50, 6, 5, "fp32"),
                                   (2, 4, 33, 4, 3, "bf16"), (4, 3, 40, 4, 3, "bf16"),
                                   (3, 3, 41, 3, 5, "u8"), (8, 6, 17, 40, 128, "bf16"),
                                   (8, 3, 40, 16, 128, "bf16"), (2, 3, 37, 2, 1024, "bf16")],
                         ids=lambda s: "x".join(map(str, s)))
def test_chunked_exchange_in_one_launch(shape):
    """Chunked exchanges on the direct path (16/8/4/2/1-byte vectors, 2-6 planes; 4 KiB
    rows, whose mode 0 takes the grouped tile order, with a padded last group) run as
    one launch of the chunked kernel: each workgroup moves its window tile through
    every plane, reading each plane back from the window before storing it to the
    output.  The output matches the oracle, and the window ends holding the last
    plane of every rank in the output's layout."""
    w, B, S, H, D, dtype = shape
    dt = {"bf16": torch.bfloat16, "fp32": torch.float32, "u8": torch.uint8}[dtype]
    e = torch.empty((), dtype=dt).element_size()
    lay = ua.ua2a_layout(w, B, S, H, D, e)
    win = torch.full((lay["window_bytes"],), 0x5A, dtype=torch.uint8, device=DEV)
    plan = ua.Plan(w, B, S, H, D, dt, window=win)
    plan.set_path(ua.UA2A_PATH_DIRECT)
    for mode in (0, 1):
        x = make_tensor(in_shape(w, B, S, H, D, mode), dtype, "bytes", 21 + mode)
        want = oracle_out(x, mode, w)
        xd = x.to(DEV)
        info = plan.describe(xd, mode, True)
        assert info["path"] == ua.UA2A_PATH_DIRECT and info["grid_dims"] == 3
        assert info["launches"] == 1 and info["chunked_form"] == ua.UA2A_CHUNKED_ONE_LAUNCH
        note(f"chunked one launch {shape} mode={mode} {info}")
        y = plan.exchange(xd, mode, True, out=poisoned(plan.out_shape(mode), dt))
        torch.cuda.synchronize()
        assert_same_bits(y, want, f"chunked one launch {shape} mode {mode}")
        last = want.view(torch.uint8).reshape(w, B, -1)[:, B - 1]
        assert torch.equal(win.cpu().reshape(w, -1), last), f"window after {shape} mode {mode}"
    plan.close()


LDS_CHUNKED_SHAPES = [
    (3, 4, 8, 3, 7, "bf16"),          # run 14 B: 2-byte pieces
    (4, 3, 64, 4, 7, "bf16"),         # run 14 B, line-aligned tiles
    (2, 5, 4, 6, 5, "fp32"),          # run 60 B, 4-byte pieces
    (2, 3, 80, 2, 12, "fp16"),        # run 24 B, spans of whole chunks
    (8, 2, 257, 8, 24, "bf16"),       # run 48 B, 8-byte pieces, odd S_local
    (2, 9, 300, 4, 16, "bf16"),       # run 64 B, 16-byte pieces, nine planes
    (3, 2, 16, 3, 5, "u8"),           # run 5 B: 1-byte pieces
    (130, 2, 8, 260, 3, "bf16"),      # more partial-chunk slots than lanes
    (1, 3, 8, 4, 7, "bf16"),          # w = 1
    (8, 4, 4096, 8, 32, "bf16"),      # run 64 B, 33 MB: thousands of tiles per plane
    (4, 4, 20000, 4, 7, "bf16"),      # run 14 B, 9 MB
    (3, 3, 7, 3, 7, "bf16"),          # plane 294 B: the output's offset moves with the plane
    (5, 2, 37, 10, 3, "u8"),          # plane 1110 B, 1-byte pieces
]


@pytest.mark.parametrize("mis", [(0, 0), (1, 1), (0, 1)], ids=["aligned", "offset", "window-off"])
@pytest.mark.parametrize("shape", LDS_CHUNKED_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_chunked_lds_in_one_launch(shape, mis):
    """Chunked exchanges on the LDS path (runs under 128 B or off the 16-byte
    grid; 16/8/4/2/1-byte pieces, 2-9 planes) run as one launch of the chunked
    LDS kernel: each workgroup fills LDS from a plane of the input, and each
    lane stores its chunks of the tile's window spans, reads them back and
    stores them to that plane of the output.  With `offset`, input, output
    and window all start one element past a 256-byte boundary, so spans begin
    and end inside 16-byte chunks; with `window-off` only the window does, so
    window chunks go to the output in pieces.  The output matches the oracle,
    and the window ends holding the last plane of every rank in the output's
    layout."""
    w, B, S, H, D, dtype = shape
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32, "u8": torch.uint8}[dtype]
    e = torch.empty((), dtype=dt).element_size()
    lay = ua.ua2a_layout(w, B, S, H, D, e)
    mis, mwe = mis[0], mis[1] * e         # input/output offset (elements), window offset (bytes)
    n, wb = lay["tensor_elems"], lay["window_bytes"]
    win = torch.full((wb + 512,), 0x5A, dtype=torch.uint8, device=DEV)
    plan = ua.Plan(w, B, S, H, D, dt, window=win[mwe:mwe + wb])
    plan.set_path(ua.UA2A_PATH_LDS)
    for mode in (0, 1):
        x = make_tensor(in_shape(w, B, S, H, D, mode), dtype, "bytes", 51 + mode)
        want = oracle_out(x, mode, w)
        xin = torch.zeros(n + 64, dtype=dt, device=DEV)
        xin[mis:mis + n] = x.reshape(-1).to(DEV)
        outbuf = poisoned((n + 64,), dt)
        xi = xin[mis:mis + n].view(in_shape(w, B, S, H, D, mode))
        yo = outbuf[mis:mis + n].view(plan.out_shape(mode))
        info = plan.describe(xi, mode, True, out=yo)
        assert info["path"] == ua.UA2A_PATH_LDS
        assert info["launches"] == 1 and info["chunked_form"] == ua.UA2A_CHUNKED_ONE_LAUNCH
        assert info["lds_planes"] == (min(B, 2) if lay["tensor_bytes"] // (w * B) % 16 == 0 else 1)
        note(f"chunked lds one launch {shape} mis={mis} mode={mode} {info}")
        plan.exchange(xi, mode, True, out=yo)
        torch.cuda.synchronize()
        assert_same_bits(yo, want, f"chunked lds one launch {shape} mis {mis} mode {mode}")
        guard = bits(outbuf.cpu())
        full = 255 if guard.dtype == torch.uint8 else POISON
        assert (guard[:mis] == full).all() and (guard[mis + n:] == full).all()
        wcpu = win.cpu()
        last = want.view(torch.uint8).reshape(w, B, -1)[:, B - 1]
        assert torch.equal(wcpu[mwe:mwe + wb].reshape(w, -1), last), f"window {shape} {mode}"
        assert (wcpu[:mwe] == 0x5A).all() and (wcpu[mwe + wb:] == 0x5A).all()
    plan.close()


def _random_lds_chunked_cases(n, seed):
    """Seeded chunked exchanges of 2-9 planes on the LDS path, bases off the
    16-byte grid: the window offset from the output by a multiple of 16
    bytes (whole 16-byte stores out) or not (pieces)."""
    rng = np.random.default_rng(seed)
    cases = []
    for c in _random_chunked_cases(n, seed):
        c.update(path="lds", mis_win=int(rng.choice([0, c["mis_out"] * c["e"], 2, 6])))
        c["mis_win"] -= c["mis_win"] % c["e"]
        cases.append(c)
    return cases


@pytest.mark.parametrize("case", _random_lds_chunked_cases(24, 5151), ids=lambda c: (
    f"w{c['w']}B{c['B']}S{c['S']}H{c['H']}D{c['D']}{c['name']}m{c['mode']}"
    f"{c['mis_in']}{c['mis_out']}{c['mis_win']}"))
def test_random_chunked_lds(case):
    w, B, S, H, D, dt = case["w"], case["B"], case["S"], case["H"], case["D"], case["dt"]
    n = w * B * S * H * D
    mode, e = case["mode"], case["e"]
    lay = ua.ua2a_layout(w, B, S, H, D, e)
    wb, mw = lay["window_bytes"], case["mis_win"]
    window = torch.full((wb + 512,), 0x3C, dtype=torch.uint8, device=DEV)
    plan = ua.Plan(w, B, S, H, D, dt, window=window[mw:mw + wb])
    plan.set_path(ua.UA2A_PATH_LDS)
    x = make_tensor(in_shape(w, B, S, H, D, mode), case["name"], "bytes", n % 6007)
    want = oracle_out(x, mode, w)
    xin = torch.zeros(n + 8, dtype=dt, device=DEV)
    xin[case["mis_in"]:case["mis_in"] + n] = x.reshape(-1).to(DEV)
    outbuf = poisoned((n + 8,), dt)
    xi = xin[case["mis_in"]:case["mis_in"] + n].view(in_shape(w, B, S, H, D, mode))
    yo = outbuf[case["mis_out"]:case["mis_out"] + n].view(plan.out_shape(mode))
    info = plan.describe(xi, mode, True, out=yo)
    if info["path"] == ua.UA2A_PATH_LDS:
        assert info["chunked_form"] == ua.UA2A_CHUNKED_ONE_LAUNCH and info["launches"] == 1
    note(f"random chunked lds {case} {info}")
    plan.exchange(xi, mode, True, out=yo)
    torch.cuda.synchronize()
    assert_same_bits(yo, want, f"random chunked lds case {case}")
    guard = bits(outbuf.cpu())
    full = 255 if guard.dtype == torch.uint8 else POISON
    assert (guard[:case["mis_out"]] == full).all() and (guard[case["mis_out"] + n:] == full).all()
    wcpu = window.cpu()
    assert (wcpu[:mw] == 0x3C).all() and (wcpu[mw + wb:] == 0x3C).all()
    last = want.view(torch.uint8).reshape(w, B, -1)[:, B - 1]
    assert torch.equal(wcpu[mw:mw + wb].reshape(w, -1), last), f"window after {case}"
    plan.close()


@pytest.mark.parametrize("shape,planes_held", [
    ((8, 4, 32768, 8, 32), 2),      # 64-byte runs, 537 MB, four planes of 134 MB, two per fill
    ((4, 3, 524287, 4, 7), 1),      # 14-byte runs, 352 MB, a plane 8 bytes off the 16-byte grid
    ((4, 5, 524288, 4, 7), 2),      # 14-byte runs, 587 MB, five planes: two stages and a single
], ids=["run64", "run14-odd-plane", "run14-five-planes"])
def test_chunked_lds_full_size(shape, planes_held):
    """Chunked exchanges on the LDS path at full size (windows larger than the
    on-package cache), both modes, against the oracle: LDS holds two planes at
    once when a plane is a multiple of 16 bytes, one otherwise."""
    w, B, S, H, D = shape
    lay = ua.ua2a_layout(w, B, S, H, D, 2)
    win = torch.empty(lay["window_bytes"], dtype=torch.uint8, device=DEV)
    plan = ua.Plan(w, B, S, H, D, torch.bfloat16, window=win)
    for mode in (0, 1):
        x = make_tensor(in_shape(w, B, S, H, D, mode), "bf16", "normal", 61 + mode)
        want = oracle_out(x, mode, w)
        xd = x.to(DEV)
        info = plan.describe(xd, mode, True)
        assert info["path"] == ua.UA2A_PATH_LDS and info["chunked_form"] == ua.UA2A_CHUNKED_ONE_LAUNCH
        assert info["lds_planes"] == planes_held
        note(f"chunked lds full size {shape} mode={mode} {info}")
        y = plan.exchange(xd, mode, True, out=poisoned(plan.out_shape(mode), torch.bfloat16))
        torch.cuda.synchronize()
        assert_same_bits(y, want, f"chunked lds full size {shape} mode {mode}")
        assert torch.equal(win.cpu().view(w, -1), want.view(torch.uint8).reshape(w, B, -1)[:, B - 1])
        del x, xd, y, want
    plan.close()


def _wide_cases(n, seed):
    """A wide seeded sweep of small exchanges (at most ~4 MB per tensor): every
    element size, 1-12 ranks, 1-6 planes, runs from 1 byte up, all paths, both
    modes, chunked or not, grid caps, and input, output and window bases off
    the 16-byte grid by independent amounts."""
    rng = np.random.default_rng(seed)
    dts = [("u8", torch.uint8), ("bf16", torch.bfloat16), ("fp32", torch.float32), ("f64", torch.float64)]
    cases = []
    for _ in range(n):
        name, dt = dts[int(rng.integers(0, len(dts)))]
        e = torch.empty((), dtype=dt).element_size()
        w, hl = int(rng.integers(1, 13)), int(rng.integers(1, 7))
        B, D = int(rng.integers(1, 7)), int(rng.integers(1, 161))
        S = max(1, min(int(rng.integers(1, 2000)), (4 << 20) // (w * B * w * hl * D * e)))
        cases.append(dict(w=w, B=B, S=S, H=w * hl, D=D, name=name, dt=dt, e=e,
                          mode=int(rng.integers(0, 2)), chunked=bool(rng.integers(0, 2)),
                          path=["auto", "direct", "lds"][int(rng.integers(0, 3))],
                          blocks=[0, 0, 0, 7, 300][int(rng.integers(0, 5))],
                          mis_in=int(rng.integers(0, 4)), mis_out=int(rng.integers(0, 4)),
                          mis_win=int(rng.integers(0, 4)) * e))
    return cases


@pytest.mark.parametrize("case", _wide_cases(160, 777), ids=lambda c: (
    f"w{c['w']}B{c['B']}S{c['S']}H{c['H']}D{c['D']}{c['name']}m{c['mode']}"
    f"{'c' if c['chunked'] else ''}{c['path']}b{c['blocks']}-{c['mis_in']}{c['mis_out']}{c['mis_win']}"))
def test_wide_random_sweep(case):
    """Each case against the oracle, with the output's guard band, and (chunked)
    the window's guard band and its last plane."""
    w, B, S, H, D, dt, e = case["w"], case["B"], case["S"], case["H"], case["D"], case["dt"], case["e"]
    n = w * B * S * H * D
    mode, chunked = case["mode"], case["chunked"]
    lay = ua.ua2a_layout(w, B, S, H, D, e)
    wb, mw = lay["window_bytes"], case["mis_win"]
    window = torch.full((wb + 256,), 0x3C, dtype=torch.uint8, device=DEV)
    plan = ua.Plan(w, B, S, H, D, dt, blocks=case["blocks"], window=window[mw:mw + wb])
    plan.set_path(PATHS[case["path"]])
    x = make_tensor(in_shape(w, B, S, H, D, mode), case["name"], "bytes", n % 8191)
    want = oracle_out(x, mode, w)
    xin = torch.zeros(n + 8, dtype=dt, device=DEV)
    xin[case["mis_in"]:case["mis_in"] + n] = x.reshape(-1).to(DEV)
    outbuf = poisoned((n + 8,), dt)
    xi = xin[case["mis_in"]:case["mis_in"] + n].view(in_shape(w, B, S, H, D, mode))
    yo = outbuf[case["mis_out"]:case["mis_out"] + n].view(plan.out_shape(mode))
    note(f"wide {case} {plan.describe(xi, mode, chunked, out=yo)}")
    plan.exchange(xi, mode, chunked, out=yo)
    torch.cuda.synchronize()
    assert_same_bits(yo, want, f"wide case {case}")
    guard = bits(outbuf.cpu())
    full = 255 if guard.dtype == torch.uint8 else POISON
    assert (guard[:case["mis_out"]] == full).all() and (guard[case["mis_out"] + n:] == full).all()
    wcpu = window.cpu()
    assert (wcpu[:mw] == 0x3C).all() and (wcpu[mw + wb:] == 0x3C).all()
    if chunked:
        last = want.view(torch.uint8).reshape(w, B, -1)[:, B - 1]
        assert torch.equal(wcpu[mw:mw + wb].reshape(w, -1), last), f"window after {case}"
    plan.close()


@pytest.mark.parametrize("shape,chunked", [((2, 1, 8, 4, 16, "bf16"), False), ((4, 3, 64, 4, 7, "bf16"), True),
                                           ((4, 4, 32, 16, 64, "fp16"), True)], ids=["tiny", "lds-chunked", "chunked"])
def test_bound_exchange_repeats_the_call(shape, chunked):
    """Plan.bind checks a call once and returns a function that re-issues it:
    new bytes written into the bound input between calls come out exchanged,
    three times in a row, in both modes."""
    w, B, S, H, D, dtype = shape
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    e = torch.empty((), dtype=dt).element_size()
    lay = ua.ua2a_layout(w, B, S, H, D, e)
    win = torch.empty(lay["window_bytes"], dtype=torch.uint8, device=DEV) if chunked else None
    plan = ua.Plan(w, B, S, H, D, dt, window=win)
    for mode in (0, 1):
        xd = torch.empty(in_shape(w, B, S, H, D, mode), dtype=dt, device=DEV)
        call = plan.bind(xd, mode, chunked)
        for rep in range(3):
            x = make_tensor(in_shape(w, B, S, H, D, mode), dtype, "bytes", 70 + 2 * rep + mode)
            xd.copy_(x.to(DEV))
            call.out.view(BITS_VIEW[e]).fill_(-1)
            note(f"bound {shape} chunked={chunked} mode={mode} rep={rep}")
            call()
            torch.cuda.synchronize()
            assert_same_bits(call.out, oracle_out(x, mode, w), f"bound {shape} mode {mode} rep {rep}")
    plan.close()
    with pytest.raises(ua.UA2AError):
        call()


# ------------------------------------------------------------- argument checks

def test_argument_checks_on_device_tensors():
    w, B, S, H, D = 2, 1, 8, 4, 16
    plan = ua.Plan(w, B, S, H, D, torch.bfloat16)
    x = torch.zeros((w, B, S, H, D), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ua.UA2AError) as e:
        ua.ua2a_exchange(plan.handle, 0, 0, x.data_ptr(), x.data_ptr() + 2, 0)
    assert e.value.code == ua.UA2A_ERR_ALIAS
    with pytest.raises(ua.UA2AError) as e:
        plan.exchange(x, 0, chunked=True)
    assert e.value.code == ua.UA2A_ERR_CAPACITY
    with pytest.raises(ua.UA2AError) as e:
        ua.ua2a_exchange(plan.handle, 0, 0, x.data_ptr() + 1, x.data_ptr() + 4096, 0)
    assert e.value.code == ua.UA2A_ERR_ALIGN
    with pytest.raises(ValueError):
        plan.exchange(x.transpose(2, 3), 0)
    with pytest.raises(TypeError):
        plan.exchange(x.float(), 0)
    assert plan.last_error() == ""
    # the plan still works after rejected calls
    y = plan.exchange(x, 0)
    torch.cuda.synchronize()
    assert (y == 0).all()
    plan.close()
