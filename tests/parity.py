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


U32 = 2.0 ** -24   # unit roundoff of fp32


def assert_y_f32(got, want64, pre64, x64, what):
    """fp32 y = sum_i pre_i x_i against the oracle's float64 y, within the gate tolerance carried through
    the stream sum: |got - y| <= (TOL_F32 + 4 (n + 1) u) * sum_i pre_i |x_i| for every element.

    The pages fix a tolerance for bf16 outputs and for the fp32 gates only. A y whose pre gates each lie
    within the gates' 1e-3 of the oracle's differs from it by at most 1e-3 * sum_i pre_i |x_i|, plus the
    fp32 rounding of the (n + 1)-term result; the fp32 mixing GEMM over K = n D terms moves the gates by
    about K u relative to the terms, so near elements where the streams cancel, y's difference is not
    small next to y itself (the floored metric then reads above 1e-3 once K passes ~10^4).
    pre64 [T, n] and x64 [T, n, D] are the oracle's gate and the decoded residual; returns the largest
    ratio of the difference to that bound (<= 1)."""
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want64, dtype=np.float64)
    n = pre64.shape[1]
    scale = np.einsum("ti,tid->td", np.abs(pre64), np.abs(x64))
    bound = (TOL_F32 + 4 * (n + 1) * U32) * scale
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    ratio = np.abs(g - w) / np.maximum(bound, 1e-300)
    worst = float(np.max(ratio)) if ratio.size else 0.0
    assert worst <= 1.0, f"{what}: difference {worst:.3f} x the propagated gate bound"
    return worst


def ulp(v, dtype):
    """Spacing of the storage format at |v| (one step up at the top of a binade, so a neighbour above is
    covered); dtype 'bf16' or 'f32'."""
    bits = 8 if dtype == "bf16" else 24
    a = np.maximum(np.abs(np.asarray(v, dtype=np.float64)) * (1.0 + 2.0 ** (1 - bits)), np.finfo(np.float32).tiny)
    _, e = np.frexp(a)
    return np.ldexp(1.0, e - bits)


def stored_interval(lo64, hi64, dtype):
    """The stored values (decoded) that round-to-nearest-even can give for any value in [lo64, hi64]: the
    rounding is monotone, so they lie between the roundings of the two ends."""
    return O.decode(O.encode(lo64, dtype), dtype), O.decode(O.encode(hi64, dtype), dtype)


def post_mix_interval(h, res, post, comb, dtype):
    """What a kernel that forms a post row as an fp32 chain (a = post_j h, then a = fma(comb_ij, x_i, a) for
    each i: n + 1 roundings, each within 2^-24 of the running magnitude) may store, against the oracle's
    float64 value rounded once. Its fp32 value lies within (n + 1) 2^-24 (|post_j h| + sum_i |comb_ij x_i|)
    of the float64 one, so its stored value lies between the roundings of the two ends of that interval:
    the oracle's own stored value except where the interval holds a rounding boundary (a near tie), where
    it may be the neighbour. Returns (o64 unrounded, the oracle's stored value, allowance, lo, hi) as
    float64 [T, n, D]."""
    n = res.shape[1]
    hv, xv = O.decode(h, dtype), O.decode(res, dtype)
    p64, c64 = np.asarray(post, np.float32).astype(np.float64), np.asarray(comb, np.float32).astype(np.float64)
    o64 = O.post_mix(hv, xv, p64, c64)
    mag = np.abs(p64)[:, :, None] * np.abs(hv)[:, None, :] + np.einsum("tij,tid->tjd", np.abs(c64), np.abs(xv))
    chain = (n + 2) * U32 * mag
    want = O.decode(O.encode(o64, dtype), dtype)
    lo, hi = stored_interval(o64 - chain, o64 + chain, dtype)
    lo, hi = np.minimum(lo, want), np.maximum(hi, want)
    return o64, want, np.maximum(hi - want, want - lo), lo, hi


def post_mix_bound(h, res, post, comb, dtype):
    """(the oracle's stored post rows, the allowance of an fp32-chain kernel's stored rows), float64."""
    _, want, allow, _, _ = post_mix_interval(h, res, post, comb, dtype)
    return want, allow


def pre_shift_bound(x_stored, allow, fn, hc_scale, bias, eps, repeat, n):
    """First-order bound on how far pre, post and comb of the pre step move when each stored input element
    x_k may differ by up to allow_k (a rounding decision of the step before): through the GEMM
    (sum_k |fn_kc| allow_k), the sum of squares (sum_k (2|x_k| + allow_k) allow_k) and so the RMS factor,
    the logits, the gates (sigma' = sigma (1 - sigma)), and Sinkhorn (its Jacobian in the logits, by central
    differences of the oracle's own Sinkhorn). Returns (dpre [T, n], dpost [T, n], dcomb [T, n, n])."""
    T = x_stored.shape[0]
    K = x_stored[0].size
    xf, af = x_stored.reshape(T, K), allow.reshape(T, K)
    z, r, m, ssq = O.pre_logits(x_stored.reshape(T, n, -1), fn, hc_scale, bias, eps)
    dm = af @ np.abs(np.asarray(fn, np.float64))
    ds = np.sum((2 * np.abs(xf) + af) * af, axis=1)
    dr = r * 0.5 * (ds / K) / (ssq / K + eps)
    alpha = np.abs(np.asarray(hc_scale, np.float64))[O.logit_groups(n)]
    dz = alpha[None, :] * (r[:, None] * dm + np.abs(m) * dr[:, None])
    sg = O.sigmoid(z[:, :2 * n])
    dgate = sg * (1 - sg) * dz[:, :2 * n]
    Z = z[:, 2 * n:].reshape(T, n, n)
    dZ = dz[:, 2 * n:].reshape(T, n, n)
    dcomb = np.zeros((T, n, n))
    hstep = 1e-6
    for k in range(n):
        for l in range(n):
            e = np.zeros((n, n))
            e[k, l] = hstep
            J = (O.sinkhorn(Z + e, repeat) - O.sinkhorn(Z - e, repeat)) / (2 * hstep)
            dcomb += np.abs(J) * dZ[:, k:k + 1, l:l + 1]
    return dgate[:, :n], dgate[:, n:], dcomb


def check_fused_tail(got_nz, got_out, h, res, post, comb, w, g, dtype, norm_eps, what):
    """The fused post + combine + RMSNorm against the float64 oracle, element by element.

    The kernel rounds two intermediates to the storage type ([P2] section 1: bf16 intermediates): the
    post rows o_j and the combined row c. It forms each from fp32 sums, the oracle from float64 sums, so
    near a rounding tie each may land on the neighbouring storage value. The check carries the interval of
    values each step may take through the rest of the computation (rounding is monotone):
      o_j:  post_mix_interval (the fp32 chain's error around the float64 value, then rounding);
      c:    sum_j w_j o_j over those intervals, widened by the fp32 chain's n roundings, then rounded;
      normalized = (c q) g, q = (mean(c^2) + eps)^-1/2: the oracle's unrounded value, widened by
            q |g| allow(c) + |normalized| dq/q (dq from allow(c) to first order, plus 2^-18 for the
            kernel's fp32 sum of squares, square root and products), then rounded.
    Every element must lie within its interval. Returns the plain relative error (Q21) of normalized (and
    of out) for the log.
    """
    n = res.shape[1]
    want_nz, want_out = O.mhc_post_combine_norm(h, res, post, comb, w, g, n=n, D=res.shape[2], dtype=dtype,
                                                norm_eps=norm_eps)
    _, o_st, allow_o, lo_o, hi_o = post_mix_interval(h, res, post, comb, dtype)
    assert np.array_equal(O.encode(o_st, dtype), want_out), "oracle: fused out differs from mhc_post"
    w64 = np.asarray(w, np.float32).astype(np.float64)
    wl = np.minimum(w64[:, :, None] * lo_o, w64[:, :, None] * hi_o).sum(axis=1)
    wh = np.maximum(w64[:, :, None] * lo_o, w64[:, :, None] * hi_o).sum(axis=1)
    chain_c = (n + 1) * U32 * np.einsum("tj,tjd->td", np.abs(w64), np.maximum(np.abs(lo_o), np.abs(hi_o)))
    c_or = O.decode(O.encode(np.einsum("tj,tjd->td", w64, o_st), dtype), dtype)
    clo, chi = stored_interval(wl - chain_c, wh + chain_c, dtype)
    allow_c = np.maximum(np.maximum(chi - c_or, c_or - clo), 0.0)
    nz64 = O.rms_norm(c_or, g, norm_eps)
    ms = np.mean(c_or * c_or, axis=1, keepdims=True)
    q = 1.0 / np.sqrt(ms + norm_eps)
    rel_q = 0.5 * np.mean(allow_c * (2 * np.abs(c_or) + allow_c), axis=1, keepdims=True) / (ms + norm_eps)
    delta = (q * np.abs(np.asarray(g, np.float64))[None, :] * allow_c
             + np.abs(nz64) * (rel_q + 2.0 ** -18))
    nlo, nhi = stored_interval(nz64 - delta, nz64 + delta, dtype)
    gn = decode(got_nz)
    assert np.all(np.isfinite(gn)), f"{what} normalized: non-finite output"
    bad = (gn < nlo) | (gn > nhi)
    assert not bad.any(), (f"{what} normalized: {int(bad.sum())} elements outside the interval of two rounding "
                           f"decisions (first at {np.argwhere(bad)[0].tolist()})")
    e_out = None
    if got_out is not None:
        go = decode(got_out)
        bad = (go < lo_o) | (go > hi_o)
        assert not bad.any(), f"{what} out: {int(bad.sum())} elements outside the fp32-chain + rounding interval"
        e_out = rel_err(got_out, want_out, "tensor")
    return rel_err(got_nz, want_nz, "tensor"), e_out
