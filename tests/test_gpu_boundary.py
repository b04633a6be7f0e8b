"""The layer boundary mhc_post_pre (post of the finished layer, then the next layer's pre) on the GPU.

Compared with the float64 oracle's composition on the same seeded inputs, and
with the two separate GPU calls. post and comb of the finished layer come from
the oracle's pre on the same residual, so comb is a genuine Sinkhorn output.
"""

import numpy as np
import pytest
import torch

import mhc_hyper_connection_pre_amd as mhc
from mhc_hyper_connection_pre_amd import workloads as W
import oracle.mhc_oracle as O
from parity import (TOL_BF16, TOL_F32, assert_close, decode, dev_tensor, host, post_mix_interval, pre_shift_bound,
                    rel_err)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _case(x):
    """Device inputs, plus the finished layer's post and comb (oracle pre of the residual with fn)."""
    s = x.spec
    post, comb, _ = O.mhc_pre(x.residual, x.fn, x.hc_scale, x.bias, n=s.n, D=s.D, dtype=s.dtype,
                              sinkhorn_repeat=s.sinkhorn_repeat, eps=s.eps)
    g = {k: dev_tensor(v) for k, v in x.arrays().items()}
    g["post_in"], g["comb_in"] = dev_tensor(post), dev_tensor(comb)
    fn2 = W.next_layer_fn(s)   # the next layer's fn
    g["fn2"] = dev_tensor(fn2)
    return g, post, comb, fn2


def _workspace(s, n_splits):
    need = mhc.mhc_pre_workspace_bytes(s.T, s.n, s.D, n_splits, 0 if s.dtype == "bf16" else 1)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    ws[:256].zero_()
    return ws


def _boundary(x, g, n_splits, ws):
    s = x.spec
    return mhc.mhc_post_pre(g["h"], g["residual"], g["post_in"], g["comb_in"], g["fn2"], g["hc_scale"], g["bias"],
                            sinkhorn_repeat=s.sinkhorn_repeat, eps=s.eps, n_splits=n_splits, workspace=ws)


def _check_oracle(x, outs, post, comb, fn2, what, tokens=None):
    """The oracle's composition (post, storage rounding, then pre on the stored out).

    out: the GPU forms post_j h + sum_i comb_ij x_i as an fp32 chain rounded once to bf16, the oracle in
    float64 rounded once, so near a rounding tie they may store neighbouring values; out must lie in the
    interval parity.post_mix_interval gives (the oracle's own value everywhere else). The next pre then
    runs on stored values that may differ by those allowances; their effect on pre', post' and comb' is
    bounded to first order (parity.pre_shift_bound, taken twice), and y' = sum_i pre_i out_i moves by at
    most sum_i (pre_i allow_i + |out_i| dpre_i). Each of post', comb' and y' must meet its Q21 tolerance
    after that propagated shift is taken off the difference.
    """
    s = x.spec
    h, res = x.h, x.residual
    out, p, c, y = (t if isinstance(t, np.ndarray) else host(t) for t in outs)
    if tokens is not None:   # tokens are independent: the oracle runs on the selected ones only
        h, res, post, comb = h[tokens], res[tokens], post[tokens], comb[tokens]
        out, p, c, y = out[tokens], p[tokens], c[tokens], y[tokens]
    o_out, o_p, o_c, o_y = O.mhc_post_pre(h, res, post, comb, fn2, x.hc_scale, x.bias, n=s.n, D=s.D,
                                          dtype=s.dtype, sinkhorn_repeat=s.sinkhorn_repeat, eps=s.eps)
    _, w_out, allow, lo, hi = post_mix_interval(h, res, post, comb, s.dtype)
    assert np.array_equal(O.encode(w_out, s.dtype), o_out)
    g_out = decode(out)
    bad = (g_out < lo) | (g_out > hi)
    assert not bad.any(), f"{what} out: {int(bad.sum())} elements outside the fp32-chain + rounding interval"
    near = int(np.count_nonzero(allow))
    differ = int(np.count_nonzero(g_out != w_out))
    dpre, dpost, dcomb = pre_shift_bound(w_out, allow, fn2, x.hc_scale, x.bias, s.eps, s.sinkhorn_repeat, s.n)
    dpre, dpost, dcomb = 2 * dpre, 2 * dpost, 2 * dcomb

    def shifted(got, want, shift, floor, tol, name):
        g_, w_ = decode(got), decode(want)
        rel = np.maximum(np.abs(g_ - w_) - shift, 0.0) / np.maximum(np.abs(w_), floor)
        e = float(np.max(rel)) if rel.size else 0.0
        assert e <= tol, f"{what} {name}: max rel err {e:.3e} beyond the propagated out rounding"
        return e

    e1 = shifted(p, o_p, dpost, 1e-6, TOL_F32, "post'")
    e2 = shifted(c, o_c, dcomb, 1e-6, TOL_F32, "comb'")
    w_y = decode(o_y)
    dy = np.einsum("ti,tid->td", O.mhc_pre(o_out, fn2, x.hc_scale, x.bias, n=s.n, D=s.D, dtype=s.dtype,
                                           sinkhorn_repeat=s.sinkhorn_repeat, eps=s.eps,
                                           intermediates=True)[3]["pre"], allow)
    dy = dy + np.einsum("ti,tid->td", dpre, np.abs(w_out))
    floor = 1e-3 * float(np.sqrt(np.mean(w_y * w_y))) if w_y.size else 1.0
    tol_y = TOL_BF16 if s.dtype == "bf16" else TOL_F32
    e3 = shifted(y, o_y, dy, floor, tol_y, "y'")
    _say(f"  {what}: out {differ} of {g_out.size} elements on the neighbouring value ({near} near ties); "
         f"post' {e1:.2e} comb' {e2:.2e} y' {e3:.2e} (plain: post' {rel_err(p, o_p, 'gate'):.2e} "
         f"comb' {rel_err(c, o_c, 'gate'):.2e} y' {rel_err(y, o_y, 'tensor'):.2e})")


FUSED = [(1, 4, 512), (31, 4, 1024), (67, 3, 1024), (130, 2, 512), (17, 1, 2048), (64, 4, 5120),
         (129, 4, 1056), (300, 3, 2240), (1100, 4, 7168),   # two generations, the second ragged
         (700, 4, 2560), (1500, 3, 6144)]
FALLBACK = [(7, 4, 264, "bf16"), (33, 4, 1032, "f32"), (5, 2, 72, "bf16"), (9, 8, 1032, "bf16"),
            (5, 8, 256, "f32")]


@pytest.mark.parametrize("T,n,D", FUSED, ids=lambda v: str(v))
def test_boundary_fused(T, n, D):
    assert mhc.mhc_post_pre_fused(T, n, D, 0, 0)
    x = W.generate(W.custom(T, n, D, "bf16", seed=T * 5 + n * 3 + D, fn_std=0.02))
    g, post, comb, fn2 = _case(x)
    ws = _workspace(x.spec, 0)
    outs = _boundary(x, g, 0, ws)
    assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], 0) == 0
    torch.cuda.synchronize()
    _check_oracle(x, outs, post, comb, fn2, f"fused T{T} n{n} D{D}")
    # the two separate calls: out bit for bit, the pre outputs to the path's rounding
    sep_out = mhc.mhc_post(g["h"], g["residual"], g["post_in"], g["comb_in"])
    sp, sc, sy = mhc.mhc_pre(sep_out, g["fn2"], g["hc_scale"], g["bias"], sinkhorn_repeat=x.spec.sinkhorn_repeat,
                             eps=x.spec.eps)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], sep_out), "boundary out differs from mhc_post"
    for u, v, k in zip(outs[1:], (sp, sc, sy), ("post", "comb", "y")):
        u = u.float().cpu().numpy().astype(np.float64)
        v = v.float().cpu().numpy().astype(np.float64)
        d = np.max(np.abs(u - v) / np.maximum(np.abs(v), 1e-3 if k == "y" else 1e-6))
        assert d <= (1e-2 if k == "y" else 1e-4), (k, d)


@pytest.mark.parametrize("stagger", ["0", "1"])
@pytest.mark.parametrize("T,n,D", [(300, 4, 2048), (67, 3, 1024), (2500, 4, 4096), (300, 4, 6144), (700, 3, 3072)],
                         ids=lambda v: str(v))
def test_boundary_both_pipelines(monkeypatch, T, n, D, stagger):
    """Either instance of the single-pass kernel (MHC_STAGGER: workgroup-synchronous, or one pipeline per
    wave) at the layer boundary, against the oracle on every token."""
    monkeypatch.setenv("MHC_STAGGER", stagger)
    x = W.generate(W.custom(T, n, D, "bf16", seed=T * 7 + n + D, fn_std=0.02))
    g, post, comb, fn2 = _case(x)
    ws = _workspace(x.spec, 0)
    outs = _boundary(x, g, 0, ws)
    assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], 0) == 0
    torch.cuda.synchronize()
    _check_oracle(x, outs, post, comb, fn2, f"stagger {stagger} T{T} n{n} D{D}")


@pytest.mark.parametrize("T,n,D,dt", FALLBACK, ids=lambda v: str(v))
def test_boundary_fallback(T, n, D, dt):
    """Shapes the single-pass kernel does not cover run mhc_post's and mhc_pre's kernels in sequence."""
    assert not mhc.mhc_post_pre_fused(T, n, D, 0, 0 if dt == "bf16" else 1)
    x = W.generate(W.custom(T, n, D, dt, seed=T + n + D, fn_std=0.05))
    g, post, comb, fn2 = _case(x)
    outs = _boundary(x, g, 0, _workspace(x.spec, 0))
    torch.cuda.synchronize()
    _check_oracle(x, outs, post, comb, fn2, f"fallback T{T} n{n} D{D} {dt}")


def test_boundary_explicit_splits_two_pass():
    x = W.generate(W.custom(70, 4, 1024, "bf16", seed=123, fn_std=0.02))
    g, post, comb, fn2 = _case(x)
    assert not mhc.mhc_post_pre_fused(70, 4, 1024, 3, 0)
    outs = _boundary(x, g, 3, _workspace(x.spec, 3))
    torch.cuda.synchronize()
    _check_oracle(x, outs, post, comb, fn2, "n_splits 3")


def test_boundary_metric_workload():
    """T = 2048, n = 4, D = 7168 in full, in the launch configuration bench.py times."""
    x = W.generate(W.spec("prefill-d7168"))
    g, post, comb, fn2 = _case(x)
    ws = _workspace(x.spec, 0)
    outs = _boundary(x, g, 0, ws)
    assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], 0) == 0
    torch.cuda.synchronize()
    _check_oracle(x, outs, post, comb, fn2, "prefill-d7168")


@pytest.mark.slow
def test_boundary_large():
    """T = 16384 (sixteen generations), residual with 1 % outliers x50, every token against the oracle (in
    chunks of 2048 tokens), with the finished layer's post and comb drawn by the workload generator."""
    s = W.spec("prefill-t16384-d7168")
    x = W.generate(s)
    assert mhc.mhc_post_pre_fused(s.T, s.n, s.D, 0, 0)
    post, comb = W.mixing_weights(s)
    fn2 = W.next_layer_fn(s)
    g = {k: dev_tensor(v) for k, v in x.arrays().items()}
    g["post_in"], g["comb_in"], g["fn2"] = dev_tensor(post), dev_tensor(comb), dev_tensor(fn2)
    ws = _workspace(s, 0)
    outs = _boundary(x, g, 0, ws)
    assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], 0) == 0
    torch.cuda.synchronize()
    del g
    outs = [host(t) for t in outs]
    for t0 in range(0, s.T, 2048):
        _check_oracle(x, outs, post, comb, fn2, f"T16384 tokens {t0}..{t0 + 2047}", tokens=np.arange(t0, t0 + 2048))
    c = outs[2].astype(np.float64)   # properties of comb' at every token
    assert np.all(c >= 0) and np.max(np.abs(c.sum(axis=1) - 1)) <= 1e-5
    del outs


def test_boundary_shares_workspace_with_pre():
    """mhc_pre and mhc_post_pre alternate on one workspace (epochs and tag regions carry over)."""
    x = W.generate(W.custom(300, 4, 2048, "bf16", seed=55, fn_std=0.02))
    g, post, comb, fn2 = _case(x)
    s = x.spec
    ws = _workspace(s, 0)
    want_pre = O.mhc_pre(x.residual, x.fn, x.hc_scale, x.bias, n=s.n, D=s.D, dtype=s.dtype,
                         sinkhorn_repeat=s.sinkhorn_repeat, eps=s.eps)
    for k in range(3):
        outs = _boundary(x, g, 0, ws)
        p, c, y = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], sinkhorn_repeat=s.sinkhorn_repeat,
                              eps=s.eps, workspace=ws)
        torch.cuda.synchronize()
        _check_oracle(x, outs, post, comb, fn2, f"boundary round {k}")
        for got, want, kind, name in zip((p, c, y), want_pre, ("gate", "gate", "tensor"), ("post", "comb", "y")):
            assert_close(host(got), want, kind, f"pre round {k} {name}")


@pytest.mark.parametrize("stagger", ["0", "1"])
def test_boundary_graph_replay(monkeypatch, stagger):
    """Captured once, replayed three times with eager calls on the same workspace in between; either kernel
    instance (MHC_STAGGER is read when the call is captured)."""
    monkeypatch.setenv("MHC_STAGGER", stagger)
    x = W.generate(W.custom(257, 4, 1024, "bf16", seed=66, fn_std=0.02))
    g, post, comb, fn2 = _case(x)
    s = x.spec
    ws = _workspace(s, 0)
    eager = [t.clone() for t in _boundary(x, g, 0, ws)]
    bufs = [torch.empty_like(t) for t in eager]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mhc.mhc_post_pre(g["h"], g["residual"], g["post_in"], g["comb_in"], g["fn2"], g["hc_scale"], g["bias"],
                         sinkhorn_repeat=s.sinkhorn_repeat, eps=s.eps, out=bufs[0], post_next=bufs[1],
                         comb_next=bufs[2], y=bufs[3], workspace=ws, stream=torch.cuda.current_stream())
    for k in range(3):
        for b in bufs:
            b.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for b, e in zip(bufs, eager):
            assert torch.equal(b, e), f"replay {k} differs from the eager call"
        _boundary(x, g, 0, ws)   # an eager call between replays
        torch.cuda.synchronize()


def test_boundary_layers_in_one_graph():
    """Decode size: eight boundary calls (a chain of layers: each call's out is the next call's residual) captured
    in one graph on one workspace, replayed three times with an eager call in between; every layer's outputs equal
    the same chain run eagerly, bit for bit."""
    T, n, D, L = 64, 4, 5120, 8
    assert mhc.mhc_post_pre_fused(T, n, D, 0, 0)
    x = W.generate(W.custom(T, n, D, "bf16", seed=77, fn_std=0.02))
    g, post, comb, fn2 = _case(x)
    s = x.spec
    ws = _workspace(s, 0)
    outs = [[torch.empty_like(g["residual"]), torch.empty_like(g["post_in"]), torch.empty_like(g["comb_in"]),
             torch.empty_like(g["h"])] for _ in range(L)]

    def chain(stream):
        res, p, c = g["residual"], g["post_in"], g["comb_in"]
        for o in outs:
            mhc.mhc_post_pre(g["h"], res, p, c, g["fn2"], g["hc_scale"], g["bias"], sinkhorn_repeat=s.sinkhorn_repeat,
                             eps=s.eps, out=o[0], post_next=o[1], comb_next=o[2], y=o[3], workspace=ws,
                             stream=stream)
            res, p, c = o[0], o[1], o[2]

    chain(torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager = [[t.clone() for t in o] for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain(torch.cuda.current_stream())
    for k in range(3):
        for o in outs:
            for t in o:
                t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for li, (o, e) in enumerate(zip(outs, eager)):
            for t, te in zip(o, e):
                assert torch.equal(t, te), f"replay {k}, layer {li} differs from the eager chain"
        _boundary(x, g, 0, ws)   # an eager call on the same workspace between replays
        torch.cuda.synchronize()


def test_boundary_errors():
    x = W.generate(W.custom(8, 4, 512, "bf16", seed=7))
    g, _, _, _ = _case(x)
    with pytest.raises(mhc.MhcError) as e:   # out over the residual
        mhc.mhc_post_pre(g["h"], g["residual"], g["post_in"], g["comb_in"], g["fn2"], g["hc_scale"], g["bias"],
                         out=g["residual"])
    assert e.value.status == -1
    r32 = g["residual"].float()
    with pytest.raises(mhc.MhcError) as e:   # single-pass asked for an fp32 residual
        mhc.mhc_post_pre(g["h"].float(), r32, g["post_in"], g["comb_in"], g["fn2"], g["hc_scale"], g["bias"],
                         n_splits=-1)
    assert e.value.status == -2
