"""The Python binding's host side that needs no GPU: a bound call (per-rank
or rank-stacked) keeps its plan alive and refuses to run once the plan is
closed."""
from __future__ import annotations

import gc
import types

import pytest
import torch

import ulysses_all_re_amd as ua


def _host_plan(w=2, B=1, S=4, H=4, D=8, dtype=torch.bfloat16):
    """A Plan on the real library whose tensors are host tensors: planning and
    describing are host-only calls, so the binding's checks run without a GPU."""
    plan = ua.Plan.__new__(ua.Plan)
    plan.w, plan.B, plan.S_local, plan.H, plan.D = w, B, S, H, D
    plan.dtype = dtype
    plan.elem_bytes = torch.empty((), dtype=dtype).element_size()
    plan.device = torch.device("cpu")
    plan.layout = ua.ua2a_layout(w, B, S, H, D, plan.elem_bytes)
    plan.window = None
    plan.handle = ua.ua2a_plan(w, B, S, H, D, plan.elem_bytes, 0, 0, 0, 0)
    return plan


def _bound(plan):
    xs = [torch.zeros(plan.in_shape(0)[1:], dtype=plan.dtype) for _ in range(plan.w)]
    outs = [torch.zeros(plan.out_shape(0)[1:], dtype=plan.dtype) for _ in range(plan.w)]
    return plan.bind_ranks(xs, 0, outs, stream=types.SimpleNamespace(cuda_stream=0))


def test_bound_call_keeps_its_plan_alive():
    call = _bound(_host_plan())        # no other reference to the plan
    gc.collect()
    assert call.plan.handle             # not destroyed with the last outside reference
    call.plan.close()


def test_bound_call_after_close_raises():
    plan = _host_plan()
    call = _bound(plan)
    plan.close()
    with pytest.raises(ua.UA2AError) as e:
        call()
    assert e.value.code == ua.UA2A_ERR_INVALID_ARG and "closed" in str(e.value)


def _bound_stacked(plan):
    x = torch.zeros(plan.in_shape(1), dtype=plan.dtype)
    out = torch.zeros(plan.out_shape(1), dtype=plan.dtype)
    return plan.bind(x, 1, out=out, stream=types.SimpleNamespace(cuda_stream=0))


def test_bound_exchange_keeps_its_plan_alive():
    call = _bound_stacked(_host_plan())
    gc.collect()
    assert call.plan.handle and call.out.shape == call.plan.out_shape(1)
    call.plan.close()


def test_bound_exchange_after_close_raises():
    plan = _host_plan()
    call = _bound_stacked(plan)
    plan.close()
    with pytest.raises(ua.UA2AError) as e:
        call()
    assert e.value.code == ua.UA2A_ERR_INVALID_ARG and "closed" in str(e.value)


def test_bind_checks_like_exchange():
    plan = _host_plan()
    with pytest.raises(ValueError):
        plan.bind(torch.zeros((1, 2, 3), dtype=plan.dtype), 0, out=torch.zeros(plan.out_shape(0), dtype=plan.dtype),
                  stream=types.SimpleNamespace(cuda_stream=0))
    x = torch.zeros(plan.in_shape(0), dtype=plan.dtype)
    with pytest.raises(ua.UA2AError) as e:       # chunked with no window: the library's own check
        plan.bind(x, 0, True, out=torch.zeros(plan.out_shape(0), dtype=plan.dtype),
                  stream=types.SimpleNamespace(cuda_stream=0))
    assert e.value.code == ua.UA2A_ERR_CAPACITY
    plan.close()
