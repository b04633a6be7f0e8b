"""Pure-Python scalar-loop twin of the mHC oracle (TEST INFRASTRUCTURE ONLY).

The same definition as ``mhc_oracle`` (see its module docstring for the
sources, [P1] sglang PR #24355 analysis sections 2-3 and [P2] sglang PR #39704
analysis section 1, and for the readings), written token by token and element
by element with ``math`` and Python floats, no numpy. It exists to pin the
vectorised oracle: a transposed einsum, a wrong axis or a broadcast slip there
shows up as a disagreement here. Tiny shapes only (T <= 4, n <= 8, D <= 16).

Inputs are nested Python lists (or anything indexable) of float64 values that
are already decoded from storage; outputs are float64 and unrounded.
"""

from __future__ import annotations

import math
import struct


def _sigmoid(u: float) -> float:
    if u < -700.0:          # e^-u would overflow; the limit is exactly 0 in float64
        return 0.0
    return 1.0 / (1.0 + math.exp(-u))


def pre_token(x, fn, hc_scale, bias, n: int, D: int, repeat: int, eps: float):
    """One token of mhc_pre. x[i][d], fn[k][c]; returns a dict of float64 values."""
    K = n * D
    N = n * (n + 2)
    flat = [x[k // D][k % D] for k in range(K)]          # stream-major
    s = 0.0
    for k in range(K):
        s += flat[k] * flat[k]
    r = 1.0 / math.sqrt(s / K + eps)
    m = []
    for c in range(N):
        acc = 0.0
        for k in range(K):
            acc += flat[k] * fn[k][c]
        m.append(acc)
    z = []
    for c in range(N):
        group = 0 if c < n else (1 if c < 2 * n else 2)
        z.append(hc_scale[group] * (r * m[c]) + bias[c])
    pre = [_sigmoid(z[i]) for i in range(n)]
    post = [_sigmoid(z[n + j]) for j in range(n)]
    # comb logits, row-major, exp after the per-row max shift
    M = []
    for i in range(n):
        row = [z[2 * n + i * n + j] for j in range(n)]
        mx = max(row)
        M.append([math.exp(v - mx) for v in row])
    for _ in range(repeat):
        for i in range(n):
            rs = 0.0
            for j in range(n):
                rs += M[i][j]
            for j in range(n):
                M[i][j] = M[i][j] / rs
        for j in range(n):
            cs = 0.0
            for i in range(n):
                cs += M[i][j]
            for i in range(n):
                M[i][j] = M[i][j] / cs
    y = []
    for d in range(D):
        acc = 0.0
        for i in range(n):
            acc += pre[i] * x[i][d]
        y.append(acc)
    return {"s": s, "r": r, "m": m, "z": z, "pre": pre, "post": post, "comb": M, "y": y}


def post_token(h, x, post, comb, n: int, D: int):
    """One token of mhc_post, float64: out[j][d]."""
    out = []
    for j in range(n):
        row = []
        for d in range(D):
            acc = post[j] * h[d]
            for i in range(n):
                acc += comb[i][j] * x[i][d]
            row.append(acc)
        out.append(row)
    return out


def combine_token(o, w, n: int, D: int):
    """Combine n (already rounded) post rows with weights w: c[d] = sum_j w[j] * o[j][d].

    The caller applies the storage rounding of c before ``rms_norm_row`` when
    it wants the fused semantics.
    """
    c = []
    for d in range(D):
        acc = 0.0
        for j in range(n):
            acc += w[j] * o[j][d]
        c.append(acc)
    return c


def rms_norm_row(c, g, eps: float):
    """RMSNorm of one row: (c[d] * (mean(c^2) + eps)^-1/2) * g[d]."""
    D = len(c)
    ss = 0.0
    for v in c:
        ss += v * v
    q = 1.0 / math.sqrt(ss / D + eps)
    return [(c[d] * q) * g[d] for d in range(D)]


def f32(v: float) -> float:
    """Round a Python float to the nearest fp32 value (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def bf16(v: float) -> float:
    """Round to fp32, then to the nearest bf16 value (ties to even), as a Python float."""
    u = struct.unpack("<I", struct.pack("<f", f32(v)))[0]
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]
