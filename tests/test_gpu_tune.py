"""Explicit single-pass tilings (n_splits = -S) against the oracle, the layer boundary at an explicit tiling
against its two calls, and one short tuner run (needs an MI355X)."""

import json

import numpy as np
import pytest
import torch

import mhc_hyper_connection_pre_amd as mhc
from mhc_hyper_connection_pre_amd import tune
from mhc_hyper_connection_pre_amd import workloads as W
import oracle.mhc_oracle as O
from parity import assert_close, dev_tensor, host

pytestmark = pytest.mark.gpu


def _inputs(T, n, D, seed):
    x = W.generate(W.custom(T, n, D, "bf16", seed=seed, fn_std=0.02))
    g = {k: dev_tensor(v) for k, v in x.arrays().items()}
    return x, g


def _ws(T, n, D, n_splits):
    need = mhc.mhc_pre_workspace_bytes(T, n, D, n_splits, 0)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    ws[:256].zero_()
    return ws


@pytest.mark.parametrize("T,n,D,S", [(300, 4, 7168, 32), (300, 4, 7168, 56), (300, 4, 7168, 112),
                                     (64, 4, 5120, 32), (64, 4, 5120, 40), (129, 2, 2048, 16),
                                     # D not a multiple of 64: rows and slices start mid-line (line-unit stores)
                                     (300, 4, 1120, 5), (300, 4, 1120, 7), (200, 3, 2016, 9)])
def test_explicit_single_pass_tiling(T, n, D, S):
    assert mhc.mhc_pre_splits(T, n, D, -S, 0) == S
    x, g = _inputs(T, n, D, seed=T + S)
    ws = _ws(T, n, D, -S)
    post, comb, y = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], n_splits=-S, workspace=ws)
    assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], -S) == 0
    torch.cuda.synchronize()
    s = x.spec
    op, oc, oy = O.mhc_pre(x.residual, x.fn, x.hc_scale, x.bias, n=n, D=D, dtype="bf16",
                           sinkhorn_repeat=s.sinkhorn_repeat, eps=s.eps)
    assert_close(host(post), op, "gate", f"S={S} post")
    assert_close(host(comb), oc, "gate", f"S={S} comb")
    assert_close(host(y), oy, "tensor", f"S={S} y")


@pytest.mark.parametrize("T,n,D,S", [(200, 4, 7168, 32), (200, 4, 7168, 56), (150, 4, 1120, 7), (257, 2, 1120, 5)])
def test_boundary_explicit_tiling_matches_its_two_calls(T, n, D, S):
    assert mhc.mhc_post_pre_fused(T, n, D, -S, 0)
    x, g = _inputs(T, n, D, seed=S)
    post_in = torch.rand((T, n), device="cuda", generator=torch.Generator(device="cuda").manual_seed(1))
    comb_in = torch.rand((T, n, n), device="cuda", generator=torch.Generator(device="cuda").manual_seed(2)) / n
    ws = _ws(T, n, D, -S)
    out, p2, c2, y2 = mhc.mhc_post_pre(g["h"], g["residual"], post_in, comb_in, g["fn"], g["hc_scale"], g["bias"],
                                       n_splits=-S, workspace=ws)
    out_ref = mhc.mhc_post(g["h"], g["residual"], post_in, comb_in)
    p_ref, c_ref, y_ref = mhc.mhc_pre(out_ref, g["fn"], g["hc_scale"], g["bias"], n_splits=-S, workspace=_ws(T, n, D, -S))
    torch.cuda.synchronize()
    for a, b, what in ((out, out_ref, "out"), (p2, p_ref, "post"), (c2, c_ref, "comb"), (y2, y_ref, "y")):
        assert np.array_equal(host(a), host(b)), what


def test_tuner_short_run(tmp_path):
    js, cpp = tmp_path / "t.json", tmp_path / "t.cpp"
    rc = tune.main(["--shapes", "4,1024", "--tokens", "64", "300", "--iters", "2", "--warmup", "1", "--rounds", "2",
                    "--json", str(js), "--cpp", str(cpp)])
    assert rc == 0
    d = json.loads(js.read_text())
    assert [e["op"] for e in d["entries"]] == ["pre", "boundary"]
    for e in d["entries"]:
        assert [p["T"] for p in e["points"]] == [64, 300]
        for p in e["points"]:
            times = p["us"]
            best = (p["best"], p["stagger"])
            assert tune.key(best) in times and all(v > 0 for v in times.values())
            assert set(times) == {tune.key(c) for c in tune.candidates(e["op"], p["T"], 4, 1024, 0)}
            # each single-pass slicing is timed in both kernel instances
            assert {k.split("/")[1] for k in times if "/" in k} == {"0", "1"}
    assert "kTable" in cpp.read_text()
