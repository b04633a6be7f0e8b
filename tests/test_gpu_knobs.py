"""The call's knobs on the GPU: hc_scale per group, sinkhorn_repeat, eps and the tail's norm_eps.

Every named workload runs hc_scale = (1, 1, 1), 20 repeats and eps = 1e-6, so a
kernel that mixed up the hc_scale groups, ignored the repeat count or placed eps
elsewhere would pass those. Here each path (single-pass, two-pass bf16 and fp32,
n = 8, the layer boundary fused and as two calls, the fused tail) runs with
other values, against the float64 oracle given the same values. Each case also
checks on the CPU that the oracle's answer for a wrong knob (groups rotated,
one repeat more, eps x10 / 10) lies outside the tolerance, so the case can tell
the right knob from a wrong one.
"""

import dataclasses

import numpy as np
import pytest
import torch

import mhc_hyper_connection_pre_amd as mhc
from mhc_hyper_connection_pre_amd import workloads as W
import oracle.mhc_oracle as O
from parity import TOL_BF16, TOL_F32, assert_close, check_fused_tail, dev_tensor, host, rel_err
from test_gpu_boundary import _boundary, _case, _check_oracle, _workspace

pytestmark = pytest.mark.gpu

# (hc_scale, sinkhorn_repeat, eps, residual_std): eps = 1e-2 with residual ~ N(0, 0.1) makes eps as large
# as the mean square, so where it goes decides the RMS factor
KNOBS = {
    "scale-R1": ((0.6, 1.4, 2.3), 1, 1e-6, 1.0),
    "scale-R2-eps1e-5": ((1.7, 0.45, 0.8), 2, 1e-5, 1.0),
    "scale-R7-eps1e-2": ((0.6, 1.4, 2.3), 7, 1e-2, 0.1),
    "scale-R50": ((1.3, 0.7, 0.4), 50, 1e-5, 1.0),
}


def _say(msg):
    print(msg, flush=True)


def _spec(T, n, D, dt, knob, seed):
    hc, R, eps, rstd = KNOBS[knob]
    return W.custom(T, n, D, dt, seed=seed, fn_std=0.05 if n < 8 else 0.03, hc_scale=hc, sinkhorn_repeat=R, eps=eps,
                    residual_std=rstd)


def _oracle(x, **over):
    s = x.spec
    hc = np.asarray(over.get("hc_scale", x.hc_scale), np.float32)
    return O.mhc_pre(x.residual, x.fn, hc, x.bias, n=s.n, D=s.D, dtype=s.dtype,
                     sinkhorn_repeat=over.get("repeat", s.sinkhorn_repeat), eps=over.get("eps", s.eps))


def _wrong_knobs_are_distinguishable(x, want):
    """The oracle's outputs under each wrong knob fail the tolerance against the right ones."""
    s = x.spec
    hc = tuple(s.hc_scale)
    wrong = {"hc_scale groups rotated": dict(hc_scale=(hc[1], hc[2], hc[0])),
             "hc_scale pre/post swapped": dict(hc_scale=(hc[1], hc[0], hc[2])),
             "one repeat more": dict(repeat=s.sinkhorn_repeat + 1),
             "eps x10": dict(eps=s.eps * 10), "eps / 10": dict(eps=s.eps / 10)}
    tol_t = TOL_BF16 if s.dtype == "bf16" else TOL_F32
    for name, over in wrong.items():
        got = _oracle(x, **over)
        e = max(rel_err(got[0], want[0], "gate") / TOL_F32, rel_err(got[1], want[1], "gate") / TOL_F32,
                rel_err(got[2], want[2], "tensor") / tol_t)
        if name == "one repeat more" and (s.n == 1 or s.sinkhorn_repeat >= 20):
            continue   # n = 1: comb = [[1]]; 20 repeats and more: converged to within rounding
        if name.startswith("eps") and s.eps < 1e-4 and s.residual_std >= 1.0:
            continue   # eps far below the mean square moves nothing beyond rounding
        assert e > 1.0, f"the case cannot tell '{name}' from the right knob (worst {e:.2f} x tolerance)"


PRE_CASES = [
    # (T, n, D, dtype, n_splits): single-pass n = 4, 3, 2, 1; two-pass bf16 and fp32; n = 8 (two tiles per wave)
    (300, 4, 7168, "bf16", -1), (129, 3, 2240, "bf16", -1), (130, 2, 512, "bf16", -1), (17, 1, 2048, "bf16", -1),
    (70, 4, 1024, "bf16", 3), (33, 4, 1032, "f32", 0), (130, 8, 1032, "bf16", 3), (9, 8, 520, "f32", 1),
]


@pytest.mark.parametrize("knob", sorted(KNOBS))
@pytest.mark.parametrize("T,n,D,dt,sp", PRE_CASES, ids=lambda v: str(v))
def test_pre_knobs(T, n, D, dt, sp, knob):
    x = W.generate(_spec(T, n, D, dt, knob, seed=T + 17 * n + D))
    s = x.spec
    want = _oracle(x)
    _wrong_knobs_are_distinguishable(x, want)
    g = {k: dev_tensor(v) for k, v in x.arrays().items()}
    need = mhc.mhc_pre_workspace_bytes(T, n, D, sp, 0 if dt == "bf16" else 1)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    ws[:256].zero_()
    post, comb, y = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], sinkhorn_repeat=s.sinkhorn_repeat,
                                eps=s.eps, n_splits=sp, workspace=ws)
    assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], sp) == 0
    torch.cuda.synchronize()
    e1 = assert_close(host(post), want[0], "gate", f"{knob} post")
    e2 = assert_close(host(comb), want[1], "gate", f"{knob} comb")
    e3 = assert_close(host(y), want[2], "tensor", f"{knob} y")
    _say(f"  {knob} T{T} n{n} D{D} {dt} S{sp}: post {e1:.2e} comb {e2:.2e} y {e3:.2e}")


@pytest.mark.parametrize("knob", sorted(KNOBS))
@pytest.mark.parametrize("T,n,D,dt", [(300, 4, 2048, "bf16"), (40, 8, 1032, "bf16")], ids=lambda v: str(v))
def test_boundary_knobs(T, n, D, dt, knob):
    """The layer boundary: one launch at n = 4 (the single-pass kernel with the post mix in registers), two
    calls in sequence at n = 8; the next layer's pre takes the knobs."""
    x = W.generate(_spec(T, n, D, dt, knob, seed=3 * T + n + D))
    s = x.spec
    assert bool(mhc.mhc_post_pre_fused(T, n, D, 0, 0)) == (n == 4)
    g, post, comb, fn2 = _case(x)
    ws = _workspace(s, 0)
    outs = _boundary(x, g, 0, ws)
    assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], 0) == 0
    torch.cuda.synchronize()
    _check_oracle(x, outs, post, comb, fn2, f"boundary {knob} T{T} n{n} D{D}")


@pytest.mark.parametrize("norm_eps", [0.5, 0.1])
@pytest.mark.parametrize("T,n,D,dt", [(32, 4, 5120, "bf16"), (9, 2, 1024, "f32"), (16, 8, 1024, "bf16")],
                         ids=lambda v: str(v))
def test_fused_tail_norm_eps(T, n, D, dt, norm_eps):
    """norm_eps near the combined row's mean square (0.5, 0.1): where the RMSNorm's eps goes matters."""
    x = W.generate(dataclasses.replace(W.custom(T, n, D, dt, seed=T + D + n, combine=True), norm_eps=norm_eps))
    s = x.spec
    op, oc, _ = _oracle(x)
    g = {k: dev_tensor(v) for k, v in x.arrays().items()}
    nz, out = mhc.mhc_post_combine_norm(g["h"], g["residual"], dev_tensor(op), dev_tensor(oc), g["combine_w"],
                                        g["norm_weight"], norm_eps=norm_eps)
    torch.cuda.synchronize()
    e, eo = check_fused_tail(host(nz), host(out), x.h, x.residual, op, oc, x.combine_w, x.norm_weight, dt, norm_eps,
                             f"norm_eps {norm_eps}")
    # the oracle at eps x10 is told apart by the same check
    with pytest.raises(AssertionError):
        check_fused_tail(O.mhc_post_combine_norm(x.h, x.residual, op, oc, x.combine_w, x.norm_weight, n=n, D=D,
                                                 dtype=dt, norm_eps=norm_eps * 10)[0], None, x.h, x.residual, op, oc,
                         x.combine_w, x.norm_weight, dt, norm_eps, "eps x10")
    _say(f"  fused tail T{T} n{n} D{D} {dt} norm_eps {norm_eps}: normalized {e:.2e} out {eo:.2e}")
