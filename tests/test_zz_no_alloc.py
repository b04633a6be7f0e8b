"""mhc_pre_static (the entry point that allocates nothing: its workspace is the library's per-GPU static scratch)
against mhc_pre with a caller workspace: the same bits, call after call, on the one shared scratch."""

import numpy as np
import pytest
import torch

import mhc_hyper_connection_pre_amd as mhc
from mhc_hyper_connection_pre_amd import workloads as W
import oracle.mhc_oracle as O
from parity import assert_close, dev_tensor, host

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _same(a, b):
    a = a.view(torch.int16) if a.dtype == torch.bfloat16 else a
    b = b.view(torch.int16) if b.dtype == torch.bfloat16 else b
    return torch.equal(a, b)


def _static_vs_workspace(T, n, D, dt, n_splits, seed, oracle=False):
    x = W.generate(W.custom(T, n, D, dt, seed=seed, fn_std=0.02))
    s = x.spec
    g = {k: dev_tensor(v) for k, v in x.arrays().items()}
    need = mhc.mhc_pre_workspace_bytes(T, n, D, n_splits, 0 if dt == "bf16" else 1)
    assert 0 < need <= mhc.MHC_PRE_STATIC_SCRATCH_BYTES
    # outputs preallocated (the caller's), prefilled with NaN so every element must be written
    outs = [torch.full((T, n), float("nan"), device="cuda"), torch.full((T, n, n), float("nan"), device="cuda"),
            torch.full((T, D), float("nan"), device="cuda", dtype=g["residual"].dtype)]
    _say(f"  mhc_pre_static T{T} n{n} D{D} {dt} n_splits {n_splits} (workspace {need} bytes)")
    got = mhc.mhc_pre_static(g["residual"], g["fn"], g["hc_scale"], g["bias"], sinkhorn_repeat=s.sinkhorn_repeat,
                             eps=s.eps, n_splits=n_splits, post=outs[0], comb=outs[1], y=outs[2])
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws[:256].zero_()
    want = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], sinkhorn_repeat=s.sinkhorn_repeat, eps=s.eps,
                       n_splits=n_splits, workspace=ws)
    torch.cuda.synchronize()
    for a, b, k in zip(got, want, ("post", "comb", "y")):
        assert _same(a, b), f"mhc_pre_static {k} differs from mhc_pre (T{T} n{n} D{D} n_splits {n_splits})"
    if oracle:
        op, oc, oy = O.mhc_pre(x.residual, x.fn, x.hc_scale, x.bias, n=n, D=D, dtype=dt,
                               sinkhorn_repeat=s.sinkhorn_repeat, eps=s.eps)
        assert_close(host(got[0]), op, "gate", "static post")
        assert_close(host(got[1]), oc, "gate", "static comb")
        assert_close(host(got[2]), oy, "tensor", "static y")


def test_static_scratch_calls_in_a_row():
    # the throughput shape (single-pass, 32 slices), then a smaller single-pass shape on the same scratch
    # (the shape marker changes, so the exchange words are cleared in-kernel), then the two-pass path, then
    # single-pass again after the two-pass call reset the marker
    _static_vs_workspace(2048, 4, 7168, "bf16", 0, seed=901, oracle=True)
    _static_vs_workspace(300, 4, 2048, "bf16", 0, seed=902, oracle=True)
    _static_vs_workspace(70, 4, 1024, "bf16", 3, seed=903)
    _static_vs_workspace(129, 3, 1024, "bf16", -1, seed=904)
    _static_vs_workspace(9, 2, 1024, "f32", 0, seed=905)


def test_static_scratch_rejects_sizes_over_the_limit():
    T, n, D = 16384, 4, 7168
    assert mhc.mhc_pre_workspace_bytes(T, n, D, 0) > mhc.MHC_PRE_STATIC_SCRATCH_BYTES
    r = torch.empty((T, n, D), dtype=torch.bfloat16, device="cuda")
    fn = torch.zeros((n * D, n * (n + 2)), device="cuda")
    with pytest.raises(mhc.MhcError) as e:
        mhc.mhc_pre_static(r, fn, torch.ones(3, device="cuda"), torch.zeros(n * (n + 2), device="cuda"))
    assert e.value.status == -4 and "32 MiB" in str(mhc.lib().mhc_last_error().decode())
