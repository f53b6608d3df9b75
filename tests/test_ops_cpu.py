"""The torch operator's host side: shape inference (fake tensors), the
scatter/gather-dim mapping and its refusals.  No GPU needed."""
from __future__ import annotations

import pytest
import torch

from ulysses_all_re_amd import ops


@pytest.mark.parametrize("w,B,S,H,D", [(2, 1, 8, 4, 16), (8, 1, 9450, 40, 128), (3, 2, 4681, 12, 80)])
def test_fake_shapes_follow_the_page(w, B, S, H, D):
    x = torch.empty((w, B, S, H, D), device="meta", dtype=torch.bfloat16)
    y = ops.all_to_all_4D(x, 2, 1, w)                    # scatter heads, gather sequence
    assert y.shape == (w, B, S * w, H // w, D) and y.dtype == x.dtype
    z = ops.all_to_all_4D(y, 1, 2, w)                    # the inverse
    assert z.shape == x.shape
    assert ops.all_to_all_4D(x, 2, 1, w, chunked=True).shape == y.shape


def test_traces_under_fake_tensor_mode():
    from torch._subclasses.fake_tensor import FakeTensorMode
    with FakeTensorMode():
        x = torch.empty((4, 2, 16, 8, 32), dtype=torch.float16)
        y = ops.exchange(x, 4, 0)
        assert y.shape == (4, 2, 64, 2, 32)


def test_refusals():
    x = torch.empty((2, 1, 8, 4, 16), device="meta")
    with pytest.raises(ValueError, match="unsupported"):
        ops.all_to_all_4D(x, 3, 1, 2)
    with pytest.raises(ValueError):
        ops.all_to_all_4D(torch.empty((3, 1, 8, 4, 16), device="meta"), 2, 1, 2)   # rank axis != w
    with pytest.raises(ValueError):
        ops.all_to_all_4D(torch.empty((2, 1, 7, 4, 16), device="meta"), 1, 2, 2)   # S not divisible
    with pytest.raises(RuntimeError, match="GPU only"):
        ops.exchange(torch.zeros((2, 1, 8, 4, 16)), 2, 0)                          # no CPU path
