"""Helpers for GPU-vs-oracle parity: host<->device transfer and the error metric.

Error metric (the pages give none): for every element,
    rel = |got - want| / max(|want|, floor)
with floor = 1e-3 * rms(want) for residual-shaped outputs (so cancellation
near zero cannot produce meaningless ratios) and 1e-6 for post/comb. The
gates are max rel <= 1e-2 for bf16 outputs and <= 1e-3 for fp32 post/comb
(and for fp32 residual-shaped outputs).
"""

import numpy as np
import torch

import oracle.mhc_oracle as O

TOL_BF16 = 1e-2
TOL_F32 = 1e-3


def dev_tensor(a, device="cuda"):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def host(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def decode(a):
    return O.decode(a, "bf16") if a.dtype == np.uint16 else np.asarray(a, dtype=np.float64)


def rel_err(got, want, kind):
    """Max relative error by the metric above; kind = 'tensor' or 'gate'."""
    g = decode(got)
    w = decode(want)
    assert g.shape == w.shape, (g.shape, w.shape)
    if g.size == 0:
        return 0.0
    assert np.all(np.isfinite(g)), "non-finite output"
    if kind == "gate":
        floor = 1e-6
    else:
        floor = max(1e-3 * float(np.sqrt(np.mean(w * w))), 1e-30)
    return float(np.max(np.abs(g - w) / np.maximum(np.abs(w), floor)))


def tol_for(a):
    return TOL_BF16 if a.dtype == np.uint16 else TOL_F32


def assert_close(got, want, kind, what):
    e = rel_err(got, want, kind)
    tol = TOL_F32 if kind == "gate" else tol_for(want)
    assert e <= tol, f"{what}: max rel err {e:.3e} > {tol:g}"
    return e
