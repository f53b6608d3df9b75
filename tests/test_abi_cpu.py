"""The real libua2a.so on the CPU: it loads, exports every entry point that
include/ua2a.h declares, and its host-only calls (layout, plan, describe,
status strings) behave -- without touching a GPU (no exchange is issued)."""
from __future__ import annotations

import os
import re
import subprocess

import pytest

import ulysses_all_re_amd as ua
from workloads import CONFIGS

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ua2a.h")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(ua2a_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ua.LIBRARY):
        from ulysses_all_re_amd import build
        build.build()
    return ua.load_library()


def test_header_declares_the_documented_entry_points():
    assert declared() == sorted(ua.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    syms = subprocess.check_output(["nm", "-D", "--defined-only", ua.LIBRARY], text=True)
    exported = {line.split()[-1] for line in syms.splitlines() if " T " in line}
    for name in declared():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_library_targets_gfx950(lib):
    # the embedded code object names its target
    assert b"gfx950" in open(ua.LIBRARY, "rb").read()


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_layout_of_the_workloads(lib, name):
    c = CONFIGS[name]
    e = {"bf16": 2, "fp16": 2, "fp32": 4}[c["dtype"]]
    lay = ua.ua2a_layout(c["w"], c["B"], c["S_local"], c["H"], c["D"], e)
    n = c["w"] * c["B"] * c["S_local"] * c["H"] * c["D"]
    assert lay["tensor_elems"] == n and lay["tensor_bytes"] == n * e
    assert lay["H_local"] == c["H"] // c["w"] and lay["S_global"] == c["S_local"] * c["w"]
    assert lay["run_bytes"] == c["H"] // c["w"] * c["D"] * e
    assert lay["window_bytes"] == n * e // c["B"]
    assert lay["moved_bytes"] == 2 * n * e


def test_host_only_calls(lib):
    # plan and describe make no device call; the pointers are never dereferenced
    h = ua.ua2a_plan(8, 1, 9450, 40, 128, 2, 0, 0, 0, 0)
    try:
        base = 1 << 40
        info = ua.ua2a_describe(h, 0, 0, base, base + (1 << 30))
        assert info["path"] == ua.UA2A_PATH_DIRECT and info["vector_bytes"] == 16
        assert info["block"] == 64 and info["launches"] == 1
        assert info["grid"] == info["tiles"] == 8 * 8 * -(-9450 * 80 // 64)   # 1 KiB tiles per slab
        assert info["grid_dims"] == 3                      # one tile per workgroup, 3-D grid
        ua.ua2a_plan_set_path(h, ua.UA2A_PATH_LDS)
        lds = ua.ua2a_describe(h, 1, 0, base, base + (1 << 30))
        assert lds["path"] == ua.UA2A_PATH_LDS and lds["grid_dims"] == 1
        with pytest.raises(ua.UA2AError) as e:
            ua.ua2a_describe(h, 0, 1, base, base + (1 << 30))
        assert e.value.code == ua.UA2A_ERR_CAPACITY
        with pytest.raises(ua.UA2AError) as e:
            ua.ua2a_describe(h, 0, 0, base, base + 16)
        assert e.value.code == ua.UA2A_ERR_ALIAS
        assert ua.ua2a_plan_last_error(h) == ""
    finally:
        ua.ua2a_destroy(h)
    with pytest.raises(ua.UA2AError) as e:
        ua.ua2a_plan(3, 1, 8, 4, 16, 2)
    assert e.value.code == ua.UA2A_ERR_SHAPE
    assert "window" in ua.ua2a_status_string(ua.UA2A_ERR_CAPACITY)


def test_grid_cap_uses_the_flat_grid(lib):
    h = ua.ua2a_plan(8, 1, 9450, 40, 128, 2, 1000)        # blocks = 1000
    try:
        info = ua.ua2a_describe(h, 0, 0, 1 << 40, (1 << 40) + (1 << 30))
        assert info["grid"] == 1000 and info["grid_dims"] == 1
    finally:
        ua.ua2a_destroy(h)


@pytest.mark.parametrize("shape,mode,path,blocks", [
    ((8, 32, 2 ** 17, 8, 256, 2), 0, ua.UA2A_PATH_AUTO, 0),     # 128 GiB, 4 KiB rows: flat grouped order
    ((8, 511, 2 ** 17, 8, 32, 2), 1, ua.UA2A_PATH_LDS, 0),      # 255 GiB through the LDS kernel
    ((8, 32, 2 ** 17, 8, 256, 2), 1, ua.UA2A_PATH_AUTO, 2 ** 31 - 1),   # huge blocks hint
])
def test_huge_launches_stay_within_a_dispatch(lib, shape, mode, path, blocks):
    """A flat launch keeps grid x block at most 2^31 work-items (a dispatch
    packet counts them in 32 bits); the kernels loop over the other tiles."""
    w, B, S, H, D, e = shape
    lay = ua.ua2a_layout(w, B, S, H, D, e)
    h = ua.ua2a_plan(w, B, S, H, D, e, blocks)
    try:
        ua.ua2a_plan_set_path(h, path)
        base = 1 << 44
        info = ua.ua2a_describe(h, mode, 0, base, base + lay["tensor_bytes"])
        assert info["grid_dims"] == 1
        assert info["tiles"] * info["block"] > 2 ** 32          # would not fit uncapped
        assert info["grid"] * info["block"] <= 2 ** 31
    finally:
        ua.ua2a_destroy(h)


@pytest.mark.parametrize("shape,blocks,dims", [
    ((16, 2 ** 21 + 1, 1, 16, 128, 2), 0, 1),    # 4 KiB rows: padding to whole groups would pass 2^32 tiles
    ((65535, 1, 1, 65535, 1, 1), 0, 3),          # 1-byte runs: a 3-D grid of 65535^2 workgroups
    ((65535, 1, 1, 65535, 1, 1), 2 ** 25, 1),    # ... or a flat grid looping over them
])
def test_tile_counts_near_2_32_are_exact(lib, shape, blocks, dims):
    """Mode 0 needs one tile per KiB of each (r, b, j) slab: the launch counts
    every one of them, in a grid the report does not truncate."""
    w, B, S, H, D, e = shape
    lay = ua.ua2a_layout(w, B, S, H, D, e)
    h = ua.ua2a_plan(w, B, S, H, D, e, blocks)
    try:
        base = 1 << 44
        info = ua.ua2a_describe(h, 0, 0, base, base + lay["tensor_bytes"])
        slab = S * lay["run_bytes"]
        assert info["path"] == ua.UA2A_PATH_DIRECT and info["grid_dims"] == dims
        assert info["tiles"] == w * w * B * -(-slab // 1024)
        if dims == 3:
            assert info["grid"] == info["tiles"] > 2 ** 31
        else:
            assert info["grid"] * info["block"] <= 2 ** 31
    finally:
        ua.ua2a_destroy(h)


@pytest.mark.parametrize("shape,mode,want", [
    ((8, 1, 16384, 8, 32, 2), 1, ua.UA2A_PATH_DIRECT),   # 64-byte runs, 67 MB a side: direct
    ((8, 1, 32768, 8, 32, 2), 1, ua.UA2A_PATH_LDS),      # 134 MB a side: LDS
    ((8, 1, 20480, 8, 32, 2), 1, ua.UA2A_PATH_LDS),      # exactly 80 MiB a side: LDS
    ((8, 1, 20479, 8, 32, 2), 1, ua.UA2A_PATH_DIRECT),   # one token less: direct
    ((8, 1, 16384, 8, 32, 2), 0, ua.UA2A_PATH_LDS),      # mode 0 keeps the LDS kernel
    ((4, 1, 2 ** 16, 4, 7, 2), 1, ua.UA2A_PATH_LDS),     # 14-byte runs: no 16-byte pieces
    ((8, 1, 9450, 40, 128, 2), 1, ua.UA2A_PATH_DIRECT),  # long runs: direct at any size
])
def test_automatic_path_by_launch_size(lib, shape, mode, want):
    """Mode 1 on short 16-byte-multiple runs takes the direct kernel below
    80 MiB a side and the LDS kernel from there on (measured crossover)."""
    w, B, S, H, D, e = shape
    lay = ua.ua2a_layout(w, B, S, H, D, e)
    h = ua.ua2a_plan(w, B, S, H, D, e, 0)
    try:
        base = 1 << 44
        info = ua.ua2a_describe(h, mode, 0, base, base + lay["tensor_bytes"])
        assert info["path"] == want, (shape, mode, info)
    finally:
        ua.ua2a_destroy(h)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(ua, "_lib", None)
    monkeypatch.setattr(ua, "LIBRARY", str(tmp_path / "libua2a.so"))
    with pytest.raises(RuntimeError, match="no non-HIP implementation"):
        ua.load_library()


def test_c_consumer_compiles_against_the_header(lib):
    """include/ua2a.h is plain C99 and libua2a.so links from C (the GPU test runs it)."""
    from tests.c_abi import build as cbuild
    path = cbuild.build()
    assert os.path.exists(path)
