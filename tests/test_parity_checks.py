"""The parity checks themselves, on the CPU: each accepts the oracle's own output and refuses a planted
mistake of the size it is meant to catch (the GPU tests rely on both)."""

import numpy as np
import pytest

from mhc_hyper_connection_pre_amd import workloads as W
import oracle.mhc_oracle as O
from parity import assert_close, assert_y_f32


@pytest.fixture(scope="module")
def f32_case():
    x = W.generate(W.custom(48, 4, 2828, "f32", seed=3, fn_std=0.02))
    out = O.mhc_pre(x.residual, x.fn, x.hc_scale, x.bias, n=4, D=2828, dtype="f32", sinkhorn_repeat=20, eps=1e-6,
                    intermediates=True)
    return x, out


def test_y_f32_check_accepts_the_stored_oracle_value(f32_case):
    x, (_, _, oy, inter) = f32_case
    r = assert_y_f32(oy, inter["y"], inter["pre"], O.decode(x.residual, "f32"), "oracle")
    assert r < 0.01   # only the fp32 storage rounding


@pytest.mark.parametrize("scale,idx", [(1.01, 0), (0.998, 2), (1.005, 3)])
def test_y_f32_check_refuses_a_wrong_gate(f32_case, scale, idx):
    x, (_, _, _, inter) = f32_case
    xr = O.decode(x.residual, "f32")
    pre = inter["pre"].copy()
    pre[:, idx] *= scale
    with pytest.raises(AssertionError):
        assert_y_f32(np.einsum("ti,tid->td", pre, xr), inter["y"], inter["pre"], xr, "planted")


def test_y_f32_check_refuses_a_dropped_stream(f32_case):
    x, (_, _, _, inter) = f32_case
    xr = O.decode(x.residual, "f32")
    pre = inter["pre"].copy()
    pre[:, 1] = 0.0
    with pytest.raises(AssertionError):
        assert_y_f32(np.einsum("ti,tid->td", pre, xr), inter["y"], inter["pre"], xr, "planted")


def test_gate_check_refuses_a_relative_error_above_its_bar(f32_case):
    _, (op, _, _, _) = f32_case
    assert_close(op, op, "gate", "self")
    with pytest.raises(AssertionError):
        assert_close(op * np.float32(1.002), op, "gate", "planted")
