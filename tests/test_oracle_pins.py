"""The float64 oracle against closed forms, exact arithmetic, invariants and brute force."""

import numpy as np
import pytest

import oracle.mhc_oracle as O
from oracle_pins import ALL_PINS
from mhc_hyper_connection_pre_amd import workloads as W


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O)


def test_invariants_tiny_workload():
    """Sinkhorn output of the tiny fp32 workload is non-negative with row and column sums 1 within 1e-4."""
    s = W.spec("tiny-f32")
    x = W.generate(s)
    post, comb, y, it = O.mhc_pre(x.residual, x.fn, x.hc_scale, x.bias, n=s.n, D=s.D, dtype=s.dtype,
                                  sinkhorn_repeat=s.sinkhorn_repeat, eps=s.eps, intermediates=True)
    assert np.all(comb >= 0)
    assert np.max(np.abs(it["comb"].sum(axis=1) - 1)) <= 1e-12
    assert np.max(np.abs(it["comb"].sum(axis=2) - 1)) <= 1e-4
    assert np.all((post > 0) & (post < 1))


def test_identity_post_returns_residual_on_workload():
    s = W.spec("decode-t32-d5120")
    x = W.generate(s)
    eye = np.broadcast_to(np.eye(s.n, dtype=np.float32), (s.T, s.n, s.n)).copy()
    out = O.mhc_post(x.h, x.residual, np.zeros((s.T, s.n), np.float32), eye, n=s.n, D=s.D, dtype=s.dtype)
    assert np.array_equal(out, x.residual)
