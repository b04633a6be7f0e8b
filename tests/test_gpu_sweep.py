"""A seeded sweep of random shapes, tilings and knobs against the oracle.

The named workloads and the targeted cases fix one axis at a time; this sweep
draws all of them at once (n, D, T, dtype, n_splits among the values the
library accepts for the shape, the single-pass kernel's instance, hc_scale,
sinkhorn_repeat, eps), for the pre step (also in long runs of generations,
T up to 8192) and for the layer boundary, so that a
combination no targeted case covers still meets the oracle. The draws are
fixed by the seed: a failure names its case and reproduces.
"""

import dataclasses

import numpy as np
import pytest
import torch

import mhc_hyper_connection_pre_amd as mhc
from mhc_hyper_connection_pre_amd import workloads as W
import oracle.mhc_oracle as O
from parity import assert_close, assert_y_f32, dev_tensor, host
from test_gpu_boundary import _boundary, _case, _check_oracle, _workspace

pytestmark = pytest.mark.gpu

SEED = 20261204


@dataclasses.dataclass(frozen=True)
class Case:
    T: int
    n: int
    D: int
    dtype: str
    hc_scale: tuple
    repeat: int
    eps: float
    pick: int       # index into the accepted n_splits values, drawn on the GPU side
    stagger: str    # the single-pass kernel's instance: "0", "1"
    seed: int

    def __str__(self):
        return (f"T{self.T}-n{self.n}-D{self.D}-{self.dtype}-R{self.repeat}-eps{self.eps:g}-"
                f"hc{'/'.join(f'{v:.2f}' for v in self.hc_scale)}-pick{self.pick}-stag{self.stagger}")


def _draw(count, boundary):
    rng = np.random.default_rng(SEED + (1 if boundary else 0))
    out = []
    while len(out) < count:
        n = int(rng.choice([1, 2, 3, 4, 4, 4, 8]))
        dtype = "bf16" if (boundary or rng.random() < 0.8) else "f32"
        if dtype == "bf16":
            # mostly multiples of 32 (the single-pass kernel's unit), some of 8 only
            D = int(32 * rng.integers(1, 225)) if rng.random() < 0.85 else int(8 * rng.integers(1, 300))
        else:
            D = int(4 * rng.integers(1, 1025))
        T = int(np.exp(rng.uniform(0.0, np.log(2500.0))))
        if T * n * D > 40_000_000:   # keep each case to a few hundred MB of host arrays
            continue
        hc = tuple(float(v) for v in rng.uniform(0.5, 2.0, size=3))
        out.append(Case(T=max(T, 1), n=n, D=D, dtype=dtype, hc_scale=hc,
                        repeat=int(rng.choice([1, 3, 7, 20])), eps=float(rng.choice([1e-6, 1e-5, 1e-3])),
                        pick=int(rng.integers(0, 1 << 20)), stagger=str(int(rng.integers(0, 2))),
                        seed=int(rng.integers(1, 1 << 30))))
    return out


PRE_CASES = _draw(96, boundary=False)
BOUNDARY_CASES = _draw(32, boundary=True)


def _draw_long(count):
    """Long runs of generations on the single-pass kernel: bf16, n <= 4, T up to 8192."""
    rng = np.random.default_rng(SEED + 2)
    out = []
    while len(out) < count:
        n = int(rng.choice([2, 3, 4, 4]))
        D = int(32 * rng.integers(8, 225))
        T = int(rng.integers(1500, 8193))
        if T * n * D > 40_000_000:
            continue
        hc = tuple(float(v) for v in rng.uniform(0.5, 2.0, size=3))
        out.append(Case(T=T, n=n, D=D, dtype="bf16", hc_scale=hc, repeat=int(rng.choice([3, 20])),
                        eps=float(rng.choice([1e-6, 1e-3])), pick=int(rng.integers(0, 1 << 20)),
                        stagger=str(int(rng.integers(0, 2))), seed=int(rng.integers(1, 1 << 30))))
    return out


LONG_CASES = _draw_long(12)


def _spec(c):
    fn_std = 0.05 if c.n < 4 else (0.02 if c.n == 4 else 0.03)
    return W.custom(c.T, c.n, c.D, c.dtype, seed=c.seed, fn_std=fn_std, hc_scale=c.hc_scale,
                    sinkhorn_repeat=c.repeat, eps=c.eps)


def _accepted_splits(T, n, D, dt, boundary):
    """n_splits values the library accepts for the shape: 0, -1 and the valid -S, and two-pass counts."""
    L = mhc.lib()
    vals = [0]
    if L.mhc_pre_splits(T, n, D, -1, dt) > 0:
        vals.append(-1)
        vals += [-S for S in range(2, 129) if L.mhc_pre_splits(T, n, D, -S, dt) == S]
    vals += [S for S in (1, 2, 3, 4, 8, 16) if L.mhc_pre_splits(T, n, D, S, dt) == S]
    if boundary:
        vals = [v for v in vals if v >= 0 or L.mhc_post_pre_fused(T, n, D, v, dt) == 1]
    return vals


def _tokens(T, seed):
    if T <= 400:
        return None
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], np.arange(max(0, T - 40), T), rng.choice(T, 48, replace=False)]))


@pytest.mark.parametrize("c", PRE_CASES + LONG_CASES, ids=str)
def test_pre_sweep(monkeypatch, c):
    monkeypatch.setenv("MHC_STAGGER", c.stagger)
    x = W.generate(_spec(c))
    dt = 0 if c.dtype == "bf16" else 1
    vals = _accepted_splits(c.T, c.n, c.D, dt, False)
    sp = vals[c.pick % len(vals)]
    g = {k: dev_tensor(v) for k, v in x.arrays().items()}
    need = mhc.mhc_pre_workspace_bytes(c.T, c.n, c.D, sp, dt)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    print(f"  {c}: n_splits {sp} (of {len(vals)} accepted)", flush=True)
    post, comb, y = mhc.mhc_pre(g["residual"], g["fn"], g["hc_scale"], g["bias"], sinkhorn_repeat=c.repeat,
                                eps=c.eps, n_splits=sp, workspace=ws)
    assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], sp) == 0
    torch.cuda.synchronize()
    tok = _tokens(c.T, c.seed)
    res = x.residual if tok is None else x.residual[tok]
    op, oc, oy, inter = O.mhc_pre(res, x.fn, x.hc_scale, x.bias, n=c.n, D=c.D, dtype=c.dtype,
                                  sinkhorn_repeat=c.repeat, eps=c.eps, intermediates=True)
    hp, hc, hy = host(post), host(comb), host(y)
    if tok is not None:
        hp, hc, hy = hp[tok], hc[tok], hy[tok]
    assert_close(hp, op, "gate", f"{c} post")
    assert_close(hc, oc, "gate", f"{c} comb")
    if c.dtype == "bf16":
        assert_close(hy, oy, "tensor", f"{c} y")
    else:   # fp32 y: the gates' tolerance carried through the stream sum
        assert_y_f32(hy, inter["y"], inter["pre"], O.decode(res, "f32"), f"{c} y")


@pytest.mark.parametrize("c", BOUNDARY_CASES, ids=str)
def test_boundary_sweep(monkeypatch, c):
    monkeypatch.setenv("MHC_STAGGER", c.stagger)
    x = W.generate(_spec(c))
    vals = _accepted_splits(c.T, c.n, c.D, 0, True)
    sp = vals[c.pick % len(vals)]
    g, post, comb, fn2 = _case(x)
    ws = _workspace(x.spec, sp)
    print(f"  {c}: n_splits {sp} (of {len(vals)} accepted), one launch "
          f"{bool(mhc.mhc_post_pre_fused(c.T, c.n, c.D, sp, 0))}", flush=True)
    outs = _boundary(x, g, sp, ws)
    assert mhc.mhc_pre_sync_timeouts(ws, g["residual"], sp) == 0
    torch.cuda.synchronize()
    _check_oracle(x, outs, post, comb, fn2, str(c), tokens=_tokens(c.T, c.seed))
