"""Pins of the float64 oracle against facts it shares no code with.

Each ``pin_*`` function takes the oracle module and raises AssertionError when
the oracle disagrees with mathematics fixed independently of it: closed forms,
exact rational arithmetic, invariants, special cases that reduce to a library
routine, and the pure-Python brute-force twin on tiny inputs. They are run
against the real oracle (test_oracle_pins.py) and against copies with planted
mistakes (test_oracle_mutations.py), where at least one pin must fail.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch

from oracle import brute as B

EPS = 1e-6


def _case(seed, T, n, D, fn_std=0.3, hc=None):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, n, D)).astype(np.float32).astype(np.float64)
    fn = g.standard_normal((n * D, n * (n + 2))) * fn_std
    bias = g.standard_normal(n * (n + 2)) * 0.3
    hc_scale = g.uniform(0.5, 2.0, 3) if hc is None else np.asarray(hc, dtype=np.float64)
    return x, fn, bias, hc_scale


def _close(a, b, rtol=1e-12, atol=1e-13, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = np.abs(a - b) - (atol + rtol * np.abs(b))
    assert np.all(err <= 0), f"{what}: max abs diff {np.max(np.abs(a - b))}"


def _pre_all(O, x, fn, hc, bias, n, R, eps=EPS):
    """Run the oracle's mhc_pre on f32-stored x and return its float64 intermediates."""
    T, _, D = x.shape
    post, comb, y, it = O.mhc_pre(x.astype(np.float32), fn, hc, bias, n=n, D=D, dtype="f32",
                                  sinkhorn_repeat=R, eps=eps, intermediates=True)
    return it


# ---------------------------------------------------------------- brute force

def pin_brute_pre(O):
    """Whole pre pipeline vs scalar loops, T <= 3, n in 1..4 and 8, D <= 8, random R."""
    g = np.random.default_rng(11)
    for case in range(18):
        n = 1 + case % 4 if case < 16 else 8
        D = (1, 2, 3, 8)[(case // 4) % 4]
        T = 1 + case % 3
        R = int(g.integers(1, 7))
        x, fn, bias, hc = _case(100 + case, T, n, D)
        it = _pre_all(O, x, fn, hc, bias, n, R)
        for t in range(T):
            b = B.pre_token(x[t].tolist(), fn.tolist(), hc.tolist(), bias.tolist(), n, D, R, EPS)
            for k in ("s", "r", "m", "z", "pre", "post", "comb", "y"):
                _close(it[k][t], b[k], what=f"brute {k} n={n} D={D} t={t}")


def pin_brute_post(O):
    """mhc_post mix vs scalar loops; orientation of comb included."""
    g = np.random.default_rng(12)
    for n in (1, 2, 3, 4, 8):
        T, D = 2, 5
        x = g.standard_normal((T, n, D))
        h = g.standard_normal((T, D))
        post = g.uniform(0, 1, (T, n))
        comb = g.uniform(0, 1, (T, n, n))
        out = O.post_mix(h, x, post, comb)
        for t in range(T):
            ref = B.post_token(h[t].tolist(), x[t].tolist(), post[t].tolist(), comb[t].tolist(), n, D)
            _close(out[t], ref, what=f"post brute n={n}")


# ---------------------------------------------------------------- rounding

def pin_rounding(O):
    """Storage rounding vs torch's own RNE conversions (library routines) and known bits."""
    g = np.random.default_rng(13)
    v = np.concatenate([g.standard_normal(20000) * 10.0 ** g.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 3.3895313892515355e38,
                         np.inf, -np.inf, 1e-40, -1e-42]])
    got = O.f64_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref), "bf16 rounding differs from torch"
    assert O.f64_to_bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80      # tie -> even
    assert O.f64_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82  # tie -> even
    assert np.isnan(O.bf16_bits_to_f64(O.f64_to_bf16_bits(np.array([np.nan]))))[0]
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    dec = O.bf16_bits_to_f64(bits)
    ref_dec = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(dec), np.isnan(ref_dec))
    ok = ~np.isnan(dec)
    assert np.array_equal(dec[ok], ref_dec[ok]), "bf16 decode differs from torch"
    f = g.standard_normal(1000)
    assert np.array_equal(O.f64_to_f32(f), torch.from_numpy(f).to(torch.float32).numpy())


# ---------------------------------------------------------------- RMS / GEMM / scale / bias

def pin_rms_closed_form(O):
    """x = c everywhere: s = n*D*c^2 and r = (c^2 + eps)^-1/2; one stream only: mean over n*D."""
    for n, D, c in ((1, 4, 1e-3), (4, 8, 0.5), (3, 5, 2.0), (2, 3, 1e-3)):
        x = np.full((1, n, D), c)
        z, r, m, s = O.pre_logits(x, np.zeros((n * D, n * (n + 2))), np.ones(3), np.zeros(n * (n + 2)), EPS)
        _close(s, [n * D * c * c], what="s")
        _close(r, [1.0 / math.sqrt(c * c + EPS)], what="r const")
        x = np.zeros((1, n, D))
        x[0, 0, :] = c
        z, r, m, s = O.pre_logits(x, np.zeros((n * D, n * (n + 2))), np.ones(3), np.zeros(n * (n + 2)), EPS)
        _close(r, [1.0 / math.sqrt(c * c / n + EPS)], what="r one stream")


def pin_gemm_onehot_and_groups(O):
    """One-hot fn columns pick x[k // D, k % D]; hc_scale groups scale pre, post, comb."""
    n, D = 3, 5
    K, N = n * D, n * (n + 2)
    x, _, _, _ = _case(21, 2, n, D)
    g = np.random.default_rng(22)
    ks = g.integers(0, K, N)
    fn = np.zeros((K, N))
    fn[ks, np.arange(N)] = 1.0
    alpha = np.array([2.0, 3.0, 5.0])
    bias = g.standard_normal(N)
    z, r, m, s = O.pre_logits(x, fn, alpha, bias, EPS)
    for t in range(2):
        for c in range(N):
            k = ks[c]
            assert m[t, c] == x[t, k // D, k % D], "one-hot GEMM column"
            grp = 0 if c < n else (1 if c < 2 * n else 2)
            _close(z[t, c], alpha[grp] * (r[t] * x[t, k // D, k % D]) + bias[c], what="z group")
    # the GEMM is a plain matrix product (library routine)
    x, fn, bias, hc = _case(23, 3, 4, 6)
    z, r, m, s = O.pre_logits(x, fn, hc, bias, EPS)
    _close(m, np.matmul(x.reshape(3, 24), fn), what="matmul")


def pin_gates(O):
    """fn = 0 makes z = bias exactly, so pre/post are the logistic function of the bias."""
    n, D = 4, 3
    bias = np.array([0.0, 1.5, -2.0, 30.0, -0.5, 0.25, 800.0, -800.0] + [0.0] * 16)
    x, _, _, _ = _case(31, 2, n, D)
    it = _pre_all(O, x, np.zeros((n * D, n * (n + 2))), np.ones(3), bias, n, 3)
    for t in range(2):
        assert np.array_equal(it["z"][t], bias)
        for i in range(n):
            assert abs(it["pre"][t, i] - 1.0 / (1.0 + math.exp(-bias[i]))) <= 1e-16
        assert it["post"][t, 2] == 1.0 and it["post"][t, 3] == 0.0
        _close(it["post"][t, :2], [1.0 / (1.0 + math.exp(0.5)), 1.0 / (1.0 + math.exp(-0.25))])
    assert it["pre"][0, 0] == 0.5


# ---------------------------------------------------------------- Sinkhorn

def _exact_sinkhorn(A, R):
    """Alternating row/column normalisation of a positive rational matrix, exactly."""
    n = len(A)
    M = [[Fraction(v) for v in row] for row in A]
    for _ in range(R):
        for i in range(n):
            s = sum(M[i])
            M[i] = [v / s for v in M[i]]
        for j in range(n):
            s = sum(M[i][j] for i in range(n))
            for i in range(n):
                M[i][j] = M[i][j] / s
    return [[float(v) for v in row] for row in M]


def pin_sinkhorn_exact(O):
    """Rational matrices A, Z = log A: comb equals exact rational Sinkhorn for R = 1, 2, 3."""
    mats = [
        [[1, 2], [3, 7]],
        [[5, 1], [1, 1]],
        [[1, 2, 3], [4, 1, 9], [2, 7, 1]],
        [[1, 1, 1, 8], [2, 3, 1, 1], [1, 5, 2, 3], [7, 1, 1, 2]],
    ]
    for A in mats:
        Z = np.log(np.array(A, dtype=np.float64))[None]
        for R in (1, 2, 3):
            _close(O.sinkhorn(Z, R)[0], _exact_sinkhorn(A, R), rtol=1e-14, atol=1e-15,
                   what=f"exact sinkhorn R={R}")


def pin_sinkhorn_closed_forms(O):
    """Constant logits -> J/n; diagonal a / off-diagonal b -> closed form; n = 2 limit."""
    for n in (1, 2, 3, 4, 5, 8):
        _close(O.sinkhorn(np.full((1, n, n), 0.7), 20)[0], np.full((n, n), 1.0 / n), rtol=1e-15)
    for n, a, b in ((3, 1.0, -0.5), (4, -2.0, 0.3), (8, 0.4, -1.1)):
        Z = np.full((1, n, n), b)
        Z[0][np.diag_indices(n)] = a
        den = math.exp(a) + (n - 1) * math.exp(b)
        ref = np.full((n, n), math.exp(b) / den)
        ref[np.diag_indices(n)] = math.exp(a) / den
        for R in (1, 5):
            _close(O.sinkhorn(Z, R)[0], ref, rtol=1e-14)
    Z = np.array([[[0.3, -1.2], [0.8, 2.0]]])
    sq = math.exp((Z[0, 0, 0] + Z[0, 1, 1] - Z[0, 0, 1] - Z[0, 1, 0]) / 2)
    c = O.sinkhorn(Z, 200)[0]
    _close([c[0, 0], c[1, 1], c[0, 1], c[1, 0]], [sq / (1 + sq), sq / (1 + sq), 1 / (1 + sq), 1 / (1 + sq)],
           rtol=1e-13)


def pin_sinkhorn_invariants(O):
    """Non-negative, columns sum to 1 (the last step), per-row shifts change nothing."""
    g = np.random.default_rng(41)
    Z = g.standard_normal((64, 4, 4)) * 1.7
    C = O.sinkhorn(Z, 20)
    assert np.all(C >= 0)
    _close(C.sum(axis=1), np.ones((64, 4)), rtol=0, atol=1e-14, what="column sums")
    C2 = O.sinkhorn(Z + g.standard_normal((64, 4, 1)) * 5, 20)
    _close(C2, C, rtol=1e-13, atol=1e-15, what="row shift")
    # a large repeat count converges: rows sum to 1 as well
    C3 = O.sinkhorn(Z, 2000)
    _close(C3.sum(axis=2), np.ones((64, 4)), rtol=0, atol=1e-9, what="row sums at convergence")


# ---------------------------------------------------------------- whole pre

def pin_pre_special_cases(O):
    """n = 1 is a gated RMS-scaled copy; fn = 0 and b = 0 give y = sum_i x_i / 2."""
    x, fn, bias, hc = _case(51, 3, 1, 7)
    it = _pre_all(O, x, fn, hc, bias, 1, 20)
    assert np.array_equal(it["comb"], np.ones((3, 1, 1)))
    for t in range(3):
        r = 1.0 / math.sqrt(float(np.sum(x[t] ** 2)) / 7 + EPS)
        gate = 1.0 / (1.0 + math.exp(-(hc[0] * (r * float(x[t, 0] @ fn[:, 0])) + bias[0])))
        _close(it["y"][t], gate * x[t, 0], rtol=1e-13, what="n=1 gated copy")
    x, _, _, _ = _case(52, 2, 4, 6)
    it = _pre_all(O, x, np.zeros((24, 24)), np.ones(3), np.zeros(24), 4, 20)
    assert np.array_equal(it["y"], 0.5 * (x[:, 0] + x[:, 1] + x[:, 2] + x[:, 3]))
    assert np.array_equal(it["comb"], np.full((2, 4, 4), 0.25))


def pin_permutation_equivariance(O):
    """Relabelling the streams permutes post, comb rows/columns; y is unchanged."""
    n, D = 4, 3
    x, fn, bias, hc = _case(61, 3, n, D)
    p = np.array([2, 0, 3, 1])
    # new stream a is old stream p[a]
    xp = x[:, p, :]
    rows = np.concatenate([np.arange(p[a] * D, p[a] * D + D) for a in range(n)])
    cols = np.concatenate([p, n + p, [2 * n + p[a] * n + p[b] for a in range(n) for b in range(n)]])
    it = _pre_all(O, x, fn, hc, bias, n, 20)
    itp = _pre_all(O, xp, fn[rows][:, cols], hc, bias[cols], n, 20)
    _close(itp["post"], it["post"][:, p], rtol=1e-12)
    _close(itp["comb"], it["comb"][:, p][:, :, p], rtol=1e-11, atol=1e-14)
    _close(itp["y"], it["y"], rtol=1e-12, atol=1e-13)


def pin_stored_outputs(O):
    """Stored outputs are the float64 results rounded once (fp32 post/comb, y in dtype)."""
    x, fn, bias, hc = _case(71, 3, 4, 8)
    xb = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    xbits = xb.view(torch.int16).numpy().view(np.uint16)
    post, comb, y, it = O.mhc_pre(xbits, fn, hc, bias, n=4, D=8, dtype="bf16", sinkhorn_repeat=20,
                                  eps=EPS, intermediates=True)
    _close(it["s"], np.sum(xb.to(torch.float64).numpy().reshape(3, 32) ** 2, axis=1), rtol=1e-15)
    assert np.array_equal(post, it["post"].astype(np.float32))
    assert np.array_equal(comb, it["comb"].astype(np.float32))
    ref = torch.from_numpy(it["y"]).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, ref)


# ---------------------------------------------------------------- post

def pin_post_identities(O):
    """comb = I, post = 0 returns the residual bit for bit; post = 1, comb = 0 returns h."""
    g = np.random.default_rng(81)
    for dtype in ("bf16", "f32"):
        T, n, D = 3, 4, 16
        x32 = g.standard_normal((T, n, D)).astype(np.float32)
        h32 = g.standard_normal((T, D)).astype(np.float32)
        if dtype == "bf16":
            x = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            h = torch.from_numpy(h32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        else:
            x, h = x32, h32
        eye = np.broadcast_to(np.eye(n, dtype=np.float32), (T, n, n)).copy()
        out = O.mhc_post(h, x, np.zeros((T, n), np.float32), eye, n=n, D=D, dtype=dtype)
        assert np.array_equal(out, x)
        out = O.mhc_post(h, x, np.ones((T, n), np.float32), np.zeros((T, n, n), np.float32), n=n, D=D, dtype=dtype)
        assert np.array_equal(out, np.broadcast_to(h[:, None, :], (T, n, D)))


def pin_post_orientation(O):
    """Only stream i* non-zero and h = 0: out_j = comb[i*, j] * x_{i*} (comb is read [in, out])."""
    n, D = 4, 5
    g = np.random.default_rng(82)
    comb = g.uniform(0.1, 1.0, (1, n, n))
    post = g.uniform(0, 1, (1, n))
    for istar in range(n):
        x = np.zeros((1, n, D))
        x[0, istar] = g.standard_normal(D)
        out = O.post_mix(np.zeros((1, D)), x, post, comb)
        for j in range(n):
            _close(out[0, j], comb[0, istar, j] * x[0, istar], rtol=1e-15)
    h = g.standard_normal((1, D))
    x = g.standard_normal((1, n, D))
    _close(O.post_mix(2 * h, x, post, comb) - O.post_mix(h, x, post, comb), post[:, :, None] * h[:, None, :],
           rtol=1e-12, atol=1e-14, what="linear in h")


# ---------------------------------------------------------------- fused post + combine + RMSNorm

def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_val(bits):
    return torch.from_numpy(np.asarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def pin_combine_norm(O):
    """One-hot w selects a stream; the norm is torch's rms_norm; the fused out is mhc_post's out bit for
    bit; brute force in float64 scalar loops with bf16 rounding of the post rows and the combined row."""
    g = np.random.default_rng(91)
    T, n, D = 3, 4, 24
    x = _bf16(g.standard_normal((T, n, D)))
    h = _bf16(g.standard_normal((T, D)))
    post = g.uniform(0, 1, (T, n)).astype(np.float32)
    comb = g.uniform(0, 0.5, (T, n, n)).astype(np.float32)
    gw = g.uniform(0.5, 1.5, D).astype(np.float32)
    for k in range(n):
        w = np.zeros((T, n), np.float32)
        w[:, k] = 1.0
        nz, out = O.mhc_post_combine_norm(h, x, post, comb, w, gw, n=n, D=D, dtype="bf16", norm_eps=EPS)
        c = _bf16_val(out[:, k])
        ref = torch.nn.functional.rms_norm(torch.from_numpy(c), (D,), torch.from_numpy(gw.astype(np.float64)), EPS)
        assert np.array_equal(nz, _bf16(ref.numpy().astype(np.float32)))
    # constant combined row: normalized = c * (c^2 + eps)^-1/2 * g; at c = 2^-10 eps matters
    for cval in (0.375, 2.0 ** -10):
        nz, _ = O.mhc_post_combine_norm(_bf16(np.zeros((1, D))), _bf16(np.full((1, n, D), cval)),
                                        np.zeros((1, n), np.float32),
                                        np.broadcast_to(np.eye(n, dtype=np.float32), (1, n, n)),
                                        np.array([[1, 0, 0, 0]], np.float32), gw, n=n, D=D, dtype="bf16",
                                        norm_eps=EPS)
        assert np.array_equal(nz[0], _bf16((cval / math.sqrt(cval * cval + EPS)) * gw.astype(np.float64)))
    # brute force: float64 scalar loops, each post row and the combined row rounded once to bf16
    w = g.uniform(0, 1, (T, n)).astype(np.float32)
    nz, out = O.mhc_post_combine_norm(h, x, post, comb, w, gw, n=n, D=D, dtype="bf16", norm_eps=EPS)
    for t in range(T):
        o = B.post_token(_bf16_val(h[t]).tolist(), _bf16_val(x[t]).tolist(), post[t].astype(np.float64).tolist(),
                         comb[t].astype(np.float64).tolist(), n, D)
        o = [[B.bf16(v) for v in row] for row in o]
        assert np.array_equal(_bf16_val(out[t]), np.array(o)), "fused out vs brute"
        c = [B.bf16(v) for v in B.combine_token(o, w[t].astype(np.float64).tolist(), n, D)]
        ref = B.rms_norm_row(c, gw.astype(np.float64).tolist(), EPS)
        assert np.array_equal(nz[t], _bf16(np.asarray(ref).astype(np.float32))), "normalized vs brute"
    # the fused call's out is mhc_post's stored result (one definition of the post rows), also at a
    # size where ties of the rounding are likely to appear
    T2, D2 = 16, 512
    x2 = _bf16(g.standard_normal((T2, n, D2)))
    h2 = _bf16(g.standard_normal((T2, D2)))
    p2 = g.uniform(0, 1, (T2, n)).astype(np.float32)
    c2 = O.sinkhorn(g.standard_normal((T2, n, n)), 20).astype(np.float32)
    w2 = g.uniform(0, 1, (T2, n)).astype(np.float32)
    g2 = g.uniform(0.5, 1.5, D2).astype(np.float32)
    nz2, out2 = O.mhc_post_combine_norm(h2, x2, p2, c2, w2, g2, n=n, D=D2, dtype="bf16", norm_eps=EPS)
    assert np.array_equal(out2, O.mhc_post(h2, x2, p2, c2, n=n, D=D2, dtype="bf16")), "fused out vs mhc_post"
    cc = _bf16(np.einsum("tj,tjd->td", w2.astype(np.float64), _bf16_val(out2)))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(_bf16_val(cc)), (D2,),
                                       torch.from_numpy(g2.astype(np.float64)), EPS)
    assert np.array_equal(nz2, _bf16(ref.numpy().astype(np.float32))), "normalized vs torch rms_norm"


# ---------------------------------------------------------------- layer boundary (post, then the next pre)

def pin_post_pre_boundary(O):
    """Scalar loops for the post mix, the bf16 storage rounding and the next pre on the stored value; and
    comb = I, post = 0 reduces the boundary to mhc_pre of the residual, bit for bit."""
    g = np.random.default_rng(91)
    R = 3
    hc = np.array([1.0, 0.7, 1.3], np.float32)
    for n in (1, 2, 3, 4):
        T, D, N = 2, 8, n * (n + 2)
        x = _bf16(g.standard_normal((T, n, D)))
        h = _bf16(g.standard_normal((T, D)))
        post = g.uniform(0, 1, (T, n)).astype(np.float32)
        comb = g.uniform(0, 1, (T, n, n)).astype(np.float32)
        fn = (g.standard_normal((n * D, N)) * 0.3).astype(np.float32)
        bias = (g.standard_normal(N) * 0.3).astype(np.float32)
        out, pn, cn, yn = O.mhc_post_pre(h, x, post, comb, fn, hc, bias, n=n, D=D, dtype="bf16",
                                         sinkhorn_repeat=R, eps=EPS)
        xv, hv = _bf16_val(x), _bf16_val(h)
        for t in range(T):
            o = B.post_token(hv[t].tolist(), xv[t].tolist(), post[t].astype(np.float64).tolist(),
                             comb[t].astype(np.float64).tolist(), n, D)
            ob = [[B.bf16(v) for v in row] for row in o]
            assert np.array_equal(_bf16_val(out[t]), np.array(ob)), f"boundary out n={n} t={t}"
            b = B.pre_token(ob, fn.astype(np.float64).tolist(), hc.astype(np.float64).tolist(),
                            bias.astype(np.float64).tolist(), n, D, R, EPS)
            _close(pn[t], [B.f32(v) for v in b["post"]], rtol=2.0 ** -23, atol=0, what=f"boundary post' n={n}")
            _close(cn[t], [[B.f32(v) for v in row] for row in b["comb"]], rtol=2.0 ** -23, atol=1e-30,
                   what=f"boundary comb' n={n}")
            _close(_bf16_val(yn[t]), [B.bf16(v) for v in b["y"]], rtol=2.0 ** -8, atol=0, what=f"boundary y' n={n}")
        eye = np.broadcast_to(np.eye(n, dtype=np.float32), (T, n, n)).copy()
        out, pn, cn, yn = O.mhc_post_pre(h, x, np.zeros((T, n), np.float32), eye, fn, hc, bias, n=n, D=D,
                                         dtype="bf16", sinkhorn_repeat=R, eps=EPS)
        p0, c0, y0 = O.mhc_pre(x, fn, hc, bias, n=n, D=D, dtype="bf16", sinkhorn_repeat=R, eps=EPS)
        assert np.array_equal(out, x) and np.array_equal(pn, p0) and np.array_equal(cn, c0)
        assert np.array_equal(yn, y0)


ALL_PINS = [
    pin_brute_pre, pin_brute_post, pin_rounding, pin_rms_closed_form, pin_gemm_onehot_and_groups,
    pin_gates, pin_sinkhorn_exact, pin_sinkhorn_closed_forms, pin_sinkhorn_invariants,
    pin_pre_special_cases, pin_permutation_equivariance, pin_stored_outputs, pin_post_identities,
    pin_post_orientation, pin_combine_norm, pin_post_pre_boundary,
]
