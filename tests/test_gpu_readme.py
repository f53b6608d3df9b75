"""The README's Python examples run as written (in order, one namespace) and
give consistent results: the round trip returns the input, the operator and
the per-rank calls and the pack/unpack pair agree with the plan's exchange,
and the credit waits end
without a time-out."""
from __future__ import annotations

import os
import re

import pytest
import torch

pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def test_readme_python_examples():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    blocks = re.findall(r"```python\n(.*?)```", open(README).read(), re.S)
    assert len(blocks) >= 4
    ns: dict = {}
    for code in blocks:
        exec(compile(code, README, "exec"), ns)
    torch.cuda.synchronize()
    x, y, z, w = ns["x"], ns["y"], ns["z"], ns["w"]
    bits = lambda t: t.view(torch.int16)
    assert torch.equal(bits(z), bits(x))
    assert torch.equal(bits(ns["plan"].exchange(x, 0)), bits(y))
    assert all(torch.equal(bits(ns["outs"][k]), bits(y[k])) for k in range(w))
    assert all(torch.equal(bits(ns["outs2"][k]), bits(y[k])) for k in range(w))
    assert int(ns["status"].item()) == 0
    assert bool((ns["credits"].cpu() == 1).all())
