"""GPU: plain C programs drive the C ABI (no Python in the exchange path);
their mode-0 outputs are compared with the oracle here.  ua2a_graph captures
exchange pairs as a HIP graph with the runtime's own capture calls and checks
every replay; its timings of replays against eager calls are printed."""
from __future__ import annotations

import json
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests.c_abi import build as cbuild

pytestmark = pytest.mark.gpu

CASES = [(4, 1, 300, 8, 64), (3, 2, 37, 6, 5)]     # as in ua2a_consumer.c


def test_c_consumer(tmp_path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binary = cbuild.BINARY if os.path.exists(cbuild.BINARY) else cbuild.build()
    print("[gpu-case] C consumer", binary, flush=True)
    res = subprocess.run([binary, str(tmp_path)], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0 and "c-abi ok" in res.stdout
    for k, (w, B, S, H, D) in enumerate(CASES):
        got = np.fromfile(tmp_path / f"case{k}_mode0.bin", dtype=np.uint32)
        x = np.arange(w * B * S * H * D, dtype=np.uint32).reshape(w, B, S, H, D)
        assert np.array_equal(got, oracle.exchange(x, 0, w).ravel()), k


GRAPH_CASES = [(2, 1, 8, 4, 16), (4, 1, 1024, 24, 128)]     # as in ua2a_graph.c (tiny, mid)


def test_c_graph_capture_and_replay(tmp_path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binary = cbuild.GRAPH_BINARY if os.path.exists(cbuild.GRAPH_BINARY) else cbuild.build("ua2a_graph")
    print("[gpu-case] C graph capture", binary, flush=True)
    res = subprocess.run([binary, str(tmp_path)], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0 and "graph ok" in res.stdout
    lines = [json.loads(x) for x in res.stdout.splitlines() if x.startswith("{")]
    assert {(x["case"], x["pairs"]) for x in lines} == {(c, p) for c in ("tiny", "mid") for p in (1, 4)}
    for x in lines:
        assert x["graph_nodes"] == x["kernels"] and x["graph_us"] > 0
    for k, (w, B, S, H, D) in enumerate(GRAPH_CASES):
        got = np.fromfile(tmp_path / f"graph{k}_mode0.bin", dtype=np.uint16)
        x = (np.arange(w * B * S * H * D, dtype=np.uint32) & 0xFFFF).astype(np.uint16).reshape(w, B, S, H, D)
        assert np.array_equal(got, oracle.exchange(x, 0, w).ravel()), k
