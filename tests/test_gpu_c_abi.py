"""GPU: a plain C program drives the C ABI (no Python in the exchange path);
its mode-0 outputs are compared with the oracle here."""
from __future__ import annotations

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
