"""HIP path vs the float64 oracle on the same seeded inputs (needs an MI355X).

Small shapes span several tiles and a ragged tail and are compared element by
element; the named workloads run at full size in the launch configuration the
benchmark times, compared in full (the 16384-token prefill too, for its own split
count and the library's; other split counts there on sampled tokens).
"""

import numpy as np
import pytest
import torch

import mhc_hyper_connection_pre_amd as mhc
from mhc_hyper_connection_pre_amd import workloads as W
import oracle.mhc_oracle as O
from parity import assert_close, check_fused_tail, dev_tensor, host

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _gpu_inputs(x):
    d = {k: dev_tensor(v) for k, v in x.arrays().items()}
    return d


def _oracle_pre(x, tokens=None):
    s = x.spec
    res = x.residual if tokens is None else x.residual[tokens]
    return O.mhc_pre(res, x.fn, x.hc_scale, x.bias, n=s.n, D=s.D, dtype=s.dtype,
                     sinkhorn_repeat=s.sinkhorn_repeat, eps=s.eps)


def _check_pre(x, g, n_splits, tokens=None, what=""):
    s = x.spec
    need = mhc.mhc_pre_workspace_bytes(s.T, s.n, s.D, n_splits, 0 if s.dtype == "bf16" else 1)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    ws[:256].zero_()   # a fresh workspace: cleared status words
    post, comb, y = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], sinkhorn_repeat=s.sinkhorn_repeat,
                                eps=s.eps, n_splits=n_splits, workspace=ws)
    assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], n_splits) == 0, f"{what}: exchange poll timed out"
    torch.cuda.synchronize()
    hp, hc, hy = host(post), host(comb), host(y)
    if tokens is not None:
        hp, hc, hy = hp[tokens], hc[tokens], hy[tokens]
    op, oc, oy = _oracle_pre(x, tokens)
    e1 = assert_close(hp, op, "gate", f"{what} post")
    e2 = assert_close(hc, oc, "gate", f"{what} comb")
    e3 = assert_close(hy, oy, "tensor", f"{what} y")
    _say(f"  {what}: post {e1:.2e} comb {e2:.2e} y {e3:.2e}")
    return post, comb, y


def _check_post(x, g, post_np, comb_np, tokens=None, what=""):
    s = x.spec
    out = mhc.mhc_post(g["h"], g["residual"], dev_tensor(post_np), dev_tensor(comb_np))
    torch.cuda.synchronize()
    ho = host(out)
    if tokens is not None:
        ho = ho[tokens]
        want = O.mhc_post(x.h[tokens], x.residual[tokens], post_np[tokens], comb_np[tokens], n=s.n, D=s.D,
                          dtype=s.dtype)
    else:
        want = O.mhc_post(x.h, x.residual, post_np, comb_np, n=s.n, D=s.D, dtype=s.dtype)
    e = assert_close(ho, want, "tensor", f"{what} out")
    _say(f"  {what}: out {e:.2e}")
    return out


# ---------------------------------------------------------------- small, ragged, every n and dtype

SMALL = [(T, n, D, dt, sp) for (T, n, D) in ((1, 4, 8), (7, 4, 264), (33, 4, 1032), (67, 3, 520),
                                             (130, 2, 2056), (17, 1, 72), (5, 4, 4104), (3, 8, 520), (66, 8, 1032))
         for dt in ("bf16", "f32") for sp in (0, 1, 3)]
# n = 8 at a shape of the tile table (bf16 entries), so n_splits = 0 takes a tabled split count
SMALL += [(40, 8, 4096, "bf16", sp) for sp in (0, 1, 3)]


@pytest.mark.parametrize("T,n,D,dt,sp", SMALL, ids=lambda v: str(v))
def test_small_pre_post(T, n, D, dt, sp):
    if dt == "f32" and D % 4:
        pytest.skip("f32 needs D % 4 == 0")
    x = W.generate(W.custom(T, n, D, dt, seed=T * 131 + n * 7 + D, fn_std=0.05))
    g = _gpu_inputs(x)
    post, comb, y = _check_pre(x, g, sp, what=f"T{T} n{n} D{D} {dt} S{sp}")
    op, oc, _ = _oracle_pre(x)
    _check_post(x, g, op, oc, what=f"T{T} n{n} D{D} {dt}")


# n = 8, bf16, from 128 tokens on: the two-pass GEMM with two 16-token tiles per wave, ragged last tile
# (T not a multiple of 32), at explicit split counts and the library's (tabled at D = 4096)
N8_TALL = [(T, 8, D, sp) for (T, D) in ((130, 1032), (161, 4096)) for sp in (0, 1, 3, 7)]


@pytest.mark.parametrize("T,n,D,sp", N8_TALL, ids=lambda v: str(v))
def test_n8_two_tiles_per_wave(T, n, D, sp):
    x = W.generate(W.custom(T, n, D, "bf16", seed=T * 3 + D + sp, fn_std=0.02))
    g = _gpu_inputs(x)
    _check_pre(x, g, sp, what=f"n8 T{T} D{D} S{sp}")


def test_n8_prefill_sampled():
    """n = 8 at T = 2048, D = 7168 (the throughput shape with eight streams), library tiling; the oracle on
    sampled tokens (first, last, both sides of every 32-token tile edge near the start, random)."""
    x = W.generate(W.custom(2048, 8, 7168, "bf16", seed=808, fn_std=0.01))
    g = _gpu_inputs(x)
    rng = np.random.default_rng(8)
    tokens = np.unique(np.concatenate([[0, 1, 31, 32, 33, 63, 64, 2047], rng.choice(2048, 56, replace=False)]))
    post, comb, _ = _check_pre(x, g, 0, tokens=tokens, what="n8 T2048 D7168")
    c = host(comb).astype(np.float64)
    assert np.all(c >= 0) and np.max(np.abs(c.sum(axis=1) - 1)) <= 1e-5


# single-pass path: bf16 with D a multiple of 128 (tiles of 128 tokens, slices of 128)
SINGLE_PASS = [(1, 4, 512), (31, 4, 1024), (33, 4, 1536), (67, 3, 1024), (130, 2, 512), (17, 1, 2048), (64, 4, 5120),
         (100, 4, 7168), (5, 4, 16384), (129, 4, 1056), (300, 3, 2240), (257, 2, 448),
         (1100, 4, 7168),   # two generations of tiles, the second one ragged
         (700, 4, 2560), (2048, 4, 6144), (1500, 3, 6144)]   # slice counts 40, 48, 24 (XCD slice runs of 5, 6, 3)


@pytest.mark.parametrize("T,n,D", SINGLE_PASS, ids=lambda v: str(v))
def test_single_pass_pre(T, n, D):
    S = mhc.mhc_pre_splits(T, n, D, -1, 0)
    assert S > 0 and D % S == 0 and (D // S) % 32 == 0
    assert mhc.mhc_pre_splits(T, n, D, 0, 0) == S   # the library's choice for bf16
    x = W.generate(W.custom(T, n, D, "bf16", seed=T * 7 + n + D, fn_std=0.02))
    g = _gpu_inputs(x)
    _check_pre(x, g, -1, what=f"single-pass T{T} n{n} D{D} S{S}")


@pytest.mark.parametrize("n_splits", [0, 3])
def test_unaligned_fn(n_splits):
    """fn at a 4-byte (not 16-byte) aligned address: the library's choice falls back to the
    two-pass path (word-wise packing loads); asking for the single-pass path is an error."""
    T, n, D = 70, 4, 1024
    x = W.generate(W.custom(T, n, D, "bf16", seed=91))
    g = _gpu_inputs(x)
    buf = torch.empty(g["fn"].numel() + 1, dtype=torch.float32, device="cuda")
    buf[1:].copy_(g["fn"].reshape(-1))
    g["fn"] = buf[1:].view(n * D, n * (n + 2))
    assert g["fn"].data_ptr() % 16 == 4
    _check_pre(x, g, n_splits, what=f"unaligned fn splits {n_splits}")
    with pytest.raises(mhc.MhcError) as e:
        mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], n_splits=-1)
    assert e.value.status == -3


def test_single_pass_matches_two_pass():
    x = W.generate(W.custom(96, 4, 4096, "bf16", seed=77))
    g = _gpu_inputs(x)
    a = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], n_splits=-1)
    b = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], n_splits=3)
    torch.cuda.synchronize()
    for u, v, k in zip(a, b, ("post", "comb", "y")):
        u = u.float().cpu().numpy().astype(np.float64)
        v = v.float().cpu().numpy().astype(np.float64)
        d = np.max(np.abs(u - v) / np.maximum(np.abs(v), 1e-3 if k == "y" else 1e-6))
        assert d <= (1e-2 if k == "y" else 1e-4), (k, d)


def _pre_into(x, g, ws, n_splits):
    s = x.spec
    return mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], sinkhorn_repeat=s.sinkhorn_repeat,
                       eps=s.eps, n_splits=n_splits, workspace=ws)


def _compare_pre(x, outs, what):
    torch.cuda.synchronize()
    op, oc, oy = _oracle_pre(x)
    assert_close(host(outs[0]), op, "gate", f"{what} post")
    assert_close(host(outs[1]), oc, "gate", f"{what} comb")
    assert_close(host(outs[2]), oy, "tensor", f"{what} y")


def test_workspace_reuse_across_shapes_and_paths():
    """One workspace serves single-pass calls of two shapes and a two-pass call in between; the
    single-pass exchange never accepts a word left by an earlier call (new inputs every call)."""
    shapes = [(300, 4, 7168), (77, 4, 4096), (300, 4, 7168), (300, 4, 7168), (77, 4, 4096)]
    splits = [-1, -1, 16, -1, -1]
    need = max(mhc.mhc_pre_workspace_bytes(T, n, D, sp, 0) for (T, n, D), sp in zip(shapes, splits))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws[:256].zero_()
    for i, ((T, n, D), sp) in enumerate(zip(shapes, splits)):
        x = W.generate(W.custom(T, n, D, "bf16", seed=400 + i))
        g = _gpu_inputs(x)
        outs = _pre_into(x, g, ws, sp)
        assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], sp) == 0
        _compare_pre(x, outs, f"reuse call {i} T{T} D{D} splits {sp}")


def test_single_pass_graph_replay():
    """The single-pass path captured in a HIP graph: every replay takes a new epoch from the
    workspace, so each replay (new inputs copied in between, eagerly) matches the oracle."""
    T, n, D = 200, 4, 7168
    xs = [W.generate(W.custom(T, n, D, "bf16", seed=500 + i)) for i in range(3)]
    g = _gpu_inputs(xs[0])
    sp = -1
    ws = torch.empty(mhc.mhc_pre_workspace_bytes(T, n, D, sp, 0), dtype=torch.uint8, device="cuda")
    ws[:256].zero_()
    post = torch.empty((T, n), dtype=torch.float32, device="cuda")
    comb = torch.empty((T, n, n), dtype=torch.float32, device="cuda")
    y = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    args = dict(sinkhorn_repeat=xs[0].spec.sinkhorn_repeat, eps=xs[0].spec.eps, n_splits=sp, workspace=ws, post=post,
                comb=comb, y=y)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], **args)   # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], **args)
    for i, x in enumerate(xs * 2):
        gi = _gpu_inputs(x)
        for k in ("residual", "fn", "hc_scale", "bias"):
            g[k].copy_(gi[k])
        graph.replay()
        torch.cuda.synchronize()
        assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], sp) == 0
        _compare_pre(x, (post, comb, y), f"graph replay {i}")


@pytest.mark.parametrize("T,n,D,dt", [(3, 4, 64, "bf16"), (65, 4, 5120, "bf16"), (9, 2, 1024, "f32"),
                                      (4, 1, 32768, "bf16"), (2, 4, 16384, "f32"), (3, 8, 64, "bf16"),
                                      (64, 8, 5120, "bf16"), (5, 8, 1024, "f32")])
def test_small_post_combine_norm(T, n, D, dt):
    x = W.generate(W.custom(T, n, D, dt, seed=5 + T + D, combine=True))
    g = _gpu_inputs(x)
    op, oc, _ = _oracle_pre(x)
    for write_out in (True, False):
        nz, out = mhc.mhc_post_combine_norm(g["h"], g["residual"], dev_tensor(op), dev_tensor(oc), g["combine_w"],
                                            g["norm_weight"], norm_eps=x.spec.norm_eps, write_out=write_out)
        torch.cuda.synchronize()
        e, eo = check_fused_tail(host(nz), host(out) if write_out else None, x.h, x.residual, op, oc, x.combine_w,
                                 x.norm_weight, dt, x.spec.norm_eps, f"T{T} n{n} D{D} {dt}")
        _say(f"  T{T} n{n} D{D} {dt} fused (out={write_out}): normalized {e:.2e} (plain metric)")


# ---------------------------------------------------------------- named workloads at full size

def test_tiny_f32_workload():
    x = W.generate(W.spec("tiny-f32"))
    s = x.spec
    g = _gpu_inputs(x)
    post, comb, y = _check_pre(x, g, s.n_splits, what="tiny-f32")
    c = host(comb).astype(np.float64)
    assert np.all(c >= 0)
    assert np.max(np.abs(c.sum(axis=1) - 1)) <= 1e-5
    assert np.max(np.abs(c.sum(axis=2) - 1)) <= 1e-4
    op, oc, _ = _oracle_pre(x)
    _check_post(x, g, op, oc, what="tiny-f32")
    nz, out = mhc.mhc_post_combine_norm(g["h"], g["residual"], dev_tensor(op), dev_tensor(oc), g["combine_w"],
                                        g["norm_weight"], norm_eps=s.norm_eps)
    torch.cuda.synchronize()
    e, eo = check_fused_tail(host(nz), host(out), x.h, x.residual, op, oc, x.combine_w, x.norm_weight, s.dtype,
                             s.norm_eps, "tiny-f32")
    assert e <= 1e-3 and eo <= 1e-3, (e, eo)


@pytest.mark.parametrize("name,n_splits", [("prefill-d4096", None), ("prefill-d7168", None), ("prefill-d7168", 16),
                                           ("prefill-d4096", 0)])
def test_prefill_workload_full(name, n_splits):
    x = W.generate(W.spec(name))
    s = x.spec
    g = _gpu_inputs(x)
    sp = s.n_splits if n_splits is None else n_splits
    post, comb, y = _check_pre(x, g, sp, what=f"{name} S{sp}")
    c = host(comb).astype(np.float64)
    assert np.all(c >= 0) and np.max(np.abs(c.sum(axis=1) - 1)) <= 1e-5
    # post at full size on the oracle's post/comb (both sides get the same inputs)
    op, oc, _ = _oracle_pre(x)
    _check_post(x, g, op, oc, what=f"{name} post")


@pytest.mark.parametrize("name", ["decode-t32-d5120", "decode-t64-d5120"])
def test_decode_workload(name):
    x = W.generate(W.spec(name))
    s = x.spec
    g = _gpu_inputs(x)
    _check_pre(x, g, s.n_splits, what=name)
    op, oc, _ = _oracle_pre(x)
    _check_post(x, g, op, oc, what=name)
    for write_out in (True, False):
        nz, out = mhc.mhc_post_combine_norm(g["h"], g["residual"], dev_tensor(op), dev_tensor(oc), g["combine_w"],
                                            g["norm_weight"], norm_eps=s.norm_eps, write_out=write_out)
        torch.cuda.synchronize()
        e, eo = check_fused_tail(host(nz), host(out) if write_out else None, x.h, x.residual, op, oc, x.combine_w,
                                 x.norm_weight, s.dtype, s.norm_eps, name)
        _say(f"  {name} fused (out={write_out}): normalized {e:.2e} (plain metric), within the rounding allowance")


_C5 = {}


def _c5():
    """The 16384-token prefill (1 % outliers x50): inputs, the oracle's pre on every token, and the oracle's
    post on seeded mixing weights, computed once for the tests that use them."""
    if not _C5:
        s = W.spec("prefill-t16384-d7168")
        x = W.generate(s)
        _C5["x"] = x
        _C5["pre"] = _oracle_pre(x)
        wp, wc = W.mixing_weights(s)
        _C5["mix"] = (wp, wc)
        _C5["out"] = O.mhc_post(x.h, x.residual, wp, wc, n=s.n, D=s.D, dtype=s.dtype)
    return _C5


@pytest.mark.slow
@pytest.mark.parametrize("n_splits", [4, 0, 2, 8])
def test_large_prefill(n_splits):
    """T = 16384: every token against the oracle for n_splits 4 (the workload's) and 0 (the library's
    choice), sampled tokens for 2 and 8; post on seeded weights for every token."""
    c5 = _c5()
    x = c5["x"]
    s = x.spec
    g = _gpu_inputs(x)
    full = n_splits in (4, 0)
    need = mhc.mhc_pre_workspace_bytes(s.T, s.n, s.D, n_splits, 0)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    ws[:256].zero_()
    post, comb, y = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], sinkhorn_repeat=s.sinkhorn_repeat,
                                eps=s.eps, n_splits=n_splits, workspace=ws)
    assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], n_splits) == 0
    torch.cuda.synchronize()
    hp, hc, hy = host(post), host(comb), host(y)
    op, oc, oy = c5["pre"]
    if not full:
        rng = np.random.default_rng(99)
        tokens = np.unique(np.concatenate([[0, 1, s.T - 1], rng.choice(s.T, 125, replace=False)]))
        hp, hc, hy, op, oc, oy = hp[tokens], hc[tokens], hy[tokens], op[tokens], oc[tokens], oy[tokens]
    e1 = assert_close(hp, op, "gate", f"T16384 S{n_splits} post")
    e2 = assert_close(hc, oc, "gate", f"T16384 S{n_splits} comb")
    e3 = assert_close(hy, oy, "tensor", f"T16384 S{n_splits} y")
    _say(f"  T16384 S{n_splits} ({'all' if full else len(hp)} tokens): post {e1:.2e} comb {e2:.2e} y {e3:.2e}")
    c = host(comb).astype(np.float64)
    assert np.all(c >= 0) and np.max(np.abs(c.sum(axis=1) - 1)) <= 1e-5
    assert np.all((host(post) > 0) & (host(post) < 1))
    del post, comb, y
    if n_splits == 4:   # post of the same workload, every token
        wp, wc = c5["mix"]
        out = mhc.mhc_post(g["h"], g["residual"], dev_tensor(wp), dev_tensor(wc))
        torch.cuda.synchronize()
        e = assert_close(host(out), c5["out"], "tensor", "T16384 out")
        _say(f"  T16384 post (all tokens): out {e:.2e}")
        del out
    del g


# ---------------------------------------------------------------- invariants, determinism, edges

def test_identity_post_is_exact():
    for dt in ("bf16", "f32"):
        x = W.generate(W.custom(37, 4, 1032, dt, seed=3))
        g = _gpu_inputs(x)
        T, n = 37, 4
        eye = torch.eye(n, device="cuda").expand(T, n, n).contiguous()
        out = mhc.mhc_post(g["h"], g["residual"], torch.zeros(T, n, device="cuda"), eye)
        assert torch.equal(out.view(torch.int16) if dt == "bf16" else out,
                           g["residual"].view(torch.int16) if dt == "bf16" else g["residual"])
        out = mhc.mhc_post(g["h"], g["residual"], torch.ones(T, n, device="cuda"),
                           torch.zeros(T, n, n, device="cuda"))
        assert torch.equal(out, g["h"][:, None, :].expand(T, n, -1))


def test_n1_is_gated_rms_scaled_copy():
    x = W.generate(W.custom(9, 1, 2048, "bf16", seed=4))
    g = _gpu_inputs(x)
    post, comb, y = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"])
    torch.cuda.synchronize()
    assert torch.equal(comb.cpu(), torch.ones(9, 1, 1))
    _, _, _, it = O.mhc_pre(x.residual, x.fn, x.hc_scale, x.bias, n=1, D=2048, dtype="bf16", sinkhorn_repeat=20,
                            eps=1e-6, intermediates=True)
    ref = it["pre"][:, 0:1] * O.decode(x.residual, "bf16")[:, 0, :]
    assert_close(host(y), O.encode(ref, "bf16"), "tensor", "n=1 y")


def test_split_invariance_and_determinism():
    x = W.generate(W.custom(300, 4, 7168, "bf16", seed=8))
    g = _gpu_inputs(x)
    res = {}
    for sp in (1, 2, 4, 8, 0, -1):
        a = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], n_splits=sp)
        b = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], n_splits=sp)
        torch.cuda.synchronize()
        for u, v in zip(a, b):
            assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                               v.view(torch.int16) if v.dtype == torch.bfloat16 else v), f"repeat differs S={sp}"
        res[sp] = [host(t) for t in a]
    for sp in (2, 4, 8, 0, -1):
        for k in (0, 1):
            d = np.max(np.abs(res[sp][k].astype(np.float64) - res[1][k]) / np.maximum(np.abs(res[1][k]), 1e-6))
            assert d <= 1e-4, (sp, k, d)


def test_outputs_fully_written_and_bounded():
    """NaN-prefilled outputs are overwritten everywhere; canaries past the end are untouched."""
    T, n, D = 45, 4, 1544
    x = W.generate(W.custom(T, n, D, "bf16", seed=12))
    g = _gpu_inputs(x)
    pad = 64
    post_b = torch.full((T * n + pad,), float("nan"), device="cuda")
    comb_b = torch.full((T * n * n + pad,), float("nan"), device="cuda")
    y_b = torch.full((T * D + pad,), float("nan"), device="cuda", dtype=torch.bfloat16)
    out_b = torch.full((T * n * D + pad,), float("nan"), device="cuda", dtype=torch.bfloat16)
    post, comb, y = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], post=post_b[:T * n].view(T, n),
                                comb=comb_b[:T * n * n].view(T, n, n), y=y_b[:T * D].view(T, D))
    out = mhc.mhc_post(g["h"], g["residual"], post, comb, out=out_b[:T * n * D].view(T, n, D))
    torch.cuda.synchronize()
    for full, used in ((post_b, T * n), (comb_b, T * n * n), (y_b, T * D), (out_b, T * n * D)):
        assert not torch.isnan(full[:used]).any()
        assert torch.isnan(full[used:]).all()


@pytest.mark.parametrize("stagger", ["0", "1"])
def test_exchange_time_out_is_reported_and_the_next_call_recovers(monkeypatch, stagger):
    # The library's poll limit is a test hook (every kernel still exits normally):
    # at -1 every exchange wait gives up whatever it reads, so every token of the
    # call is lost; at 0 every wait that its first read does not satisfy gives up
    # (a fresh workspace's grid barrier among them). MHC_STAGGER picks the kernel
    # instance: workgroup-synchronous (0) or one pipeline per wave (1).
    monkeypatch.setenv("MHC_STAGGER", stagger)
    x = W.generate(W.custom(300, 4, 1024, "bf16", seed=11))
    g = _gpu_inputs(x)
    s = x.spec
    op, oc, oy = _oracle_pre(x)
    need = mhc.mhc_pre_workspace_bytes(s.T, s.n, s.D, -1)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")

    def call():
        return mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], sinkhorn_repeat=s.sinkhorn_repeat,
                           eps=s.eps, n_splits=-1, workspace=ws)

    def lost_tokens(post, comb, y):
        hp, hc, hy = host(post), host(comb), O.decode(host(y), "bf16")
        return (np.isnan(hp).any(axis=1) | np.isnan(hc).reshape(s.T, -1).any(axis=1) | np.isnan(hy).any(axis=1),
                hp, hc, host(y))

    monkeypatch.setenv("MHC_POLL_TICKS", "-1")
    _say("  every wait gives up (poll limit -1)")
    out = call()
    assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], -1) == 1
    lost, hp, hc, hy = lost_tokens(*out)
    assert lost.all(), f"{int((~lost).sum())} tokens of a call whose every wait gave up are not NaN"
    assert np.isnan(hp).all() and np.isnan(hc).all() and np.isnan(O.decode(hy, "bf16")).all()

    monkeypatch.setenv("MHC_POLL_TICKS", "0")
    _say("  waits give up after their first read (poll limit 0)")
    out = call()
    assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], -1) == 1
    lost, hp, hc, hy = lost_tokens(*out)
    _say(f"  {int(lost.sum())} of {s.T} tokens NaN")
    if (~lost).any():   # every token is NaN or right
        assert_close(hp[~lost], op[~lost], "gate", "post of completed tokens")
        assert_close(hc[~lost], oc[~lost], "gate", "comb of completed tokens")
        assert_close(hy[~lost], oy[~lost], "tensor", "y of completed tokens")
    monkeypatch.delenv("MHC_POLL_TICKS")

    # the next call on the same workspace is a normal one
    post, comb, y = call()
    assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], -1) == 0
    assert_close(host(post), op, "gate", "post after a timed-out call")
    assert_close(host(comb), oc, "gate", "comb after a timed-out call")
    assert_close(host(y), oy, "tensor", "y after a timed-out call")


PIPELINE_CASES = [
    # (T, n, D): ragged tails, every n of the single-pass path, several generations
    (300, 4, 7168), (129, 3, 2240), (1000, 2, 512), (17, 1, 2048), (2500, 4, 4096),
    # three and six columns per slice (D = 3072 and 6144 at 32 slices)
    (700, 3, 3072), (300, 4, 6144), (2048, 4, 6144),
]


@pytest.mark.parametrize("stagger", ["0", "1"])
@pytest.mark.parametrize("T,n,D", PIPELINE_CASES, ids=lambda v: str(v))
def test_both_pipelines(monkeypatch, T, n, D, stagger):
    """The single-pass kernel has two instances, chosen by the number of generations: the workgroup
    finalises its tile's tokens together, or (from four generations on) every wave runs its own pipeline
    and finalises its own tokens. MHC_STAGGER forces either at any size; both must match the oracle."""
    monkeypatch.setenv("MHC_STAGGER", stagger)
    x = W.generate(W.custom(T, n, D, "bf16", seed=T + n + D, fn_std=0.05 if n < 4 else 0.02))
    g = _gpu_inputs(x)
    tokens = None if T <= 1000 else np.unique(np.concatenate([[0, T - 1], np.arange(T - 130, T),
                                                             np.random.default_rng(3).choice(T, 64, replace=False)]))
    _check_pre(x, g, -1, tokens, f"stagger {stagger} T{T} n{n} D{D}")


def test_side_stream_without_workspace():
    """Calls on a side stream with the binding allocating the outputs and the workspace: they are allocated
    and cleared on that stream, so memory another stream allocates meanwhile is never theirs."""
    x = W.generate(W.custom(300, 4, 2048, "bf16", seed=31, fn_std=0.02))
    s = x.spec
    g = _gpu_inputs(x)
    op, oc, oy = _oracle_pre(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    results = []
    for k in range(4):
        res = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], sinkhorn_repeat=s.sinkhorn_repeat,
                          eps=s.eps, stream=side)
        out = mhc.mhc_post(g["h"], g["residual"], res[0], res[1], stream=side)
        results.append((res, out))
        # the current stream allocates and writes memory while the side stream's calls run
        junk = torch.full((1 << 22,), float(k), device="cuda")
        junk.add_(1.0)
        del junk
    side.synchronize()
    for k, ((p, c, y), out) in enumerate(results):
        assert_close(host(p), op, "gate", f"side stream {k} post")
        assert_close(host(c), oc, "gate", f"side stream {k} comb")
        assert_close(host(y), oy, "tensor", f"side stream {k} y")
        assert_close(host(out), O.mhc_post(x.h, x.residual, host(p), host(c), n=s.n, D=s.D, dtype=s.dtype),
                     "tensor", f"side stream {k} out")


def test_default_workspace_kept_per_stream():
    """Calls that pass no workspace share one the binding keeps per (device, launch stream): a later call,
    of the same shape or another, on the same stream reuses it (one launch, no fill) and matches the same
    call with a fresh workspace of its own bit for bit; another stream gets its own; a call needing more
    room replaces it; release_workspaces() drops them."""
    mhc.release_workspaces()
    xa = W.generate(W.custom(300, 4, 2048, "bf16", seed=51, fn_std=0.02))
    xb = W.generate(W.custom(64, 4, 5120, "bf16", seed=52, fn_std=0.02))
    ga, gb = _gpu_inputs(xa), _gpu_inputs(xb)

    def pre(g, **kw):
        return mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], **kw)

    def boundary(g, p, c, **kw):
        return mhc.mhc_post_pre(g["h"], g["residual"], p, c, g["fn"], g["hc_scale"], g["bias"], **kw)

    def fresh(x):
        s = x.spec
        return torch.zeros(max(mhc.mhc_pre_workspace_bytes(s.T, s.n, s.D), 256), dtype=torch.uint8, device="cuda")

    def same(a, b, what):
        for k, (u, v) in enumerate(zip(a, b)):
            assert torch.equal(u, v), f"{what}: output {k} differs from the call with its own workspace"

    ref_a = pre(ga, workspace=fresh(xa))
    ref_b = pre(gb, workspace=fresh(xb))
    ref_ba = boundary(gb, ref_b[0], ref_b[1], workspace=fresh(xb))
    cur = torch.cuda.current_stream()
    for k in range(2):
        same(pre(ga), ref_a, f"pre A, call {k}")
    key = (torch.cuda.current_device(), cur.cuda_stream)
    assert list(mhc._WORKSPACES) == [key]
    ws0 = mhc._WORKSPACES[key]
    same(pre(gb), ref_b, "pre B after A")
    same(boundary(gb, ref_b[0], ref_b[1]), ref_ba, "boundary B")
    same(pre(ga), ref_a, "pre A after B")
    need_a = mhc.mhc_pre_workspace_bytes(300, 4, 2048)
    need_b = mhc.mhc_pre_workspace_bytes(64, 4, 5120)
    if need_b <= need_a:
        assert mhc._WORKSPACES[key] is ws0, "a call that fits reuses the stream's workspace"
    assert mhc._WORKSPACES[key].numel() >= max(need_a, need_b)
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    res = pre(ga, stream=side)
    side.synchronize()
    same(res, ref_a, "pre A on a side stream")
    assert len(mhc._WORKSPACES) == 2
    mhc.release_workspaces()
    assert not mhc._WORKSPACES
    same(pre(ga), ref_a, "pre A after release")
    mhc.release_workspaces()


def test_two_streams_with_their_own_workspaces():
    """Two single-pass calls in flight at once on two streams, each with its own workspace, sized so that
    both grids fit on the chip together (80 + 64 workgroups): neither waits for the other, and each meets
    the oracle (the exchange words of one call never reach the other's workspace)."""
    xa = W.generate(W.custom(64, 4, 5120, "bf16", seed=41, fn_std=0.02))
    xb = W.generate(W.custom(100, 3, 2048, "bf16", seed=42, fn_std=0.05))
    cases = []
    for x in (xa, xb):
        s = x.spec
        need = mhc.mhc_pre_workspace_bytes(s.T, s.n, s.D, -1)
        assert mhc.mhc_pre_splits(s.T, s.n, s.D, -1) * ((s.T + 127) // 128) <= 128
        cases.append((x, _gpu_inputs(x), torch.zeros(need, dtype=torch.uint8, device="cuda")))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    outs = []
    for k in range(3):
        for (x, g, ws), st in zip(cases, streams):
            s = x.spec
            outs.append(mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], n_splits=-1, workspace=ws,
                                    stream=st))
    for st in streams:
        st.synchronize()
    for k, (p, c, y) in enumerate(outs):
        x, g, ws = cases[k % 2]
        op, oc, oy = _oracle_pre(x)
        assert_close(host(p), op, "gate", f"stream {k % 2} call {k // 2} post")
        assert_close(host(c), oc, "gate", f"stream {k % 2} call {k // 2} comb")
        assert_close(host(y), oy, "tensor", f"stream {k % 2} call {k // 2} y")
    for x, g, ws in cases:
        assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], -1) == 0


def test_prepared_calls_repeat_the_direct_calls():
    # A PreparedCall checks and marshals once; each call launches the same entry point with the same
    # arguments, so its outputs are the direct call's bits, call after call.
    x = W.generate(W.custom(96, 4, 1024, "bf16", seed=21))
    g = _gpu_inputs(x)
    s = x.spec
    post0, comb0, y0 = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], sinkhorn_repeat=s.sinkhorn_repeat,
                                   eps=s.eps)
    h = g["h"]
    out0 = mhc.mhc_post(h, g["residual"], post0, comb0)
    pp = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], sinkhorn_repeat=s.sinkhorn_repeat, eps=s.eps,
                     prepare=True)
    pq = mhc.mhc_post(h, g["residual"], pp.outputs[0], pp.outputs[1], prepare=True)
    cw = torch.sigmoid(torch.randn((96, 4), device="cuda"))
    nw = torch.rand(1024, device="cuda") + 0.5
    n0, o0 = mhc.mhc_post_combine_norm(h, g["residual"], post0, comb0, cw, nw)
    pc = mhc.mhc_post_combine_norm(h, g["residual"], post0, comb0, cw, nw, prepare=True)
    b0 = mhc.mhc_post_pre(h, g["residual"], post0, comb0, g["fn"], g["hc_scale"], g["bias"],
                          sinkhorn_repeat=s.sinkhorn_repeat, eps=s.eps)
    pb = mhc.mhc_post_pre(h, g["residual"], post0, comb0, g["fn"], g["hc_scale"], g["bias"],
                          sinkhorn_repeat=s.sinkhorn_repeat, eps=s.eps, prepare=True)
    for _ in range(3):
        p1, c1, y1 = pp()
        o1 = pq()
        n1, oo1 = pc()
        b1 = pb()
        torch.cuda.synchronize()
        assert torch.equal(p1, post0) and torch.equal(c1, comb0) and torch.equal(y1, y0)
        assert torch.equal(o1, out0)
        assert torch.equal(n1, n0) and torch.equal(oo1, o0)
        assert all(torch.equal(u, v) for u, v in zip(b1, b0))


def test_error_paths_on_gpu():
    x = W.generate(W.custom(8, 4, 64, "bf16", seed=2))
    g = _gpu_inputs(x)
    big = torch.empty(8 * 4 * 64 + 8, dtype=torch.bfloat16, device="cuda")
    mis = big[1:1 + 8 * 4 * 64].view(8, 4, 64)
    with pytest.raises(mhc.MhcError) as e:
        mhc.mhc_pre(mis, g["fn"], g["hc_scale"], g["bias"])
    assert e.value.status == -3
    with pytest.raises(mhc.MhcError) as e:
        mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"],
                    workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    assert e.value.status == -4
    # n = 8 runs on the two-pass kernels only; n = 5 is not built
    x8 = W.generate(W.custom(4, 8, 64, "bf16", seed=3))
    g8 = _gpu_inputs(x8)
    with pytest.raises(mhc.MhcError) as e:
        mhc.mhc_pre(g8["residual"], g8["fn"], g8["hc_scale"], g8["bias"], n_splits=-1)
    assert e.value.status == -2
    x5 = W.generate(W.custom(4, 5, 64, "bf16", seed=3))
    g5 = _gpu_inputs(x5)
    with pytest.raises(mhc.MhcError) as e:
        mhc.mhc_pre(g5["residual"], g5["fn"], g5["hc_scale"], g5["bias"])
    assert e.value.status == -2
    # outputs over an input are refused before any launch
    y_in_res = g["residual"].view(-1)[:8 * 64].view(8, 64)
    with pytest.raises(mhc.MhcError) as e:
        mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], y=y_in_res)
    assert e.value.status == -1
    h = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    pin, cin = torch.full((8, 4), 0.5, device="cuda"), torch.full((8, 4, 4), 0.25, device="cuda")
    out = torch.empty((8, 4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mhc.MhcError) as e:
        mhc.mhc_post_pre(h, g["residual"], pin, cin, g["fn"], g["hc_scale"], g["bias"], out=out,
                         y=out.view(-1)[8 * 64:16 * 64].view(8, 64))
    assert e.value.status == -1
    with pytest.raises(mhc.MhcError) as e:
        mhc.mhc_post(h, g["residual"], pin, cin, out=g["residual"])
    assert e.value.status == -1
    # the binding refuses a workspace the kernels could not use
    with pytest.raises(ValueError, match="workspace"):
        mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], workspace=torch.zeros(1 << 20, dtype=torch.uint8))
    # a workspace of another element type counts its bytes
    need = mhc.mhc_pre_workspace_bytes(8, 4, 64)
    ws32 = torch.zeros((need + 3) // 4 + 64, dtype=torch.float32, device="cuda")
    p32, c32, y32 = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], workspace=ws32)
    p8, c8, y8 = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"])
    assert torch.equal(p32, p8) and torch.equal(c32, c8) and torch.equal(y32, y8)
    # T = 0 is a no-op
    z = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    p, c, y = mhc.mhc_pre(z, g["fn"], g["hc_scale"], g["bias"])
    assert p.shape == (0, 4) and y.shape == (0, 64)
