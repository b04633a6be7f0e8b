"""Float64 numpy oracle for mHC pre/post mixing (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this module. It shares no code with the HIP library and imports nothing from it.

Sources (web pages on the subject; cited by title and section):

* [P1] "[sglang] AMD ROCm DeepSeek-V4 performance optimisation: Aiter MHC kernel
  integration analysis" (sglang PR #24355). Section 2, "DeepSeek-V4 model-layer
  kernel swap", shows the layer calling ``mhc_pre(residual, fn, hc_scale, ...,
  sinkhorn_repeat)`` which returns ``(post, comb, y)`` and then
  ``mhc_post(result, x, residual, post, comb)`` into a result shaped like the
  residual. Section 3, "TileLang kernel tuning", shows the pre step as a
  split-K GEMM fused with a sum of squares. The closing "why this is a good
  optimisation" list says the fused kernel covers the Sinkhorn iterations and
  the normalisation.
* [P2] "[sglang] DeepSeek-V4.1 performance optimisation: mHC and metadata
  overhead analysis" (sglang PR #39704). Section 1, "mHC Post/Combine/RMSNorm
  fusion (prefill)", fuses the post mix with the next layer's combine into a
  bf16 ``collapsed`` buffer followed by an RMSNorm; section 2, "All-reduce
  kernel extension and fusion", returns that combined row as ``normalized``.

The computation, token by token (x is the token's residual, n streams of D):

1. s = sum of x^2 over all n*D elements; r = 1/sqrt(s/(n*D) + eps)       (RMS)
2. m = x_flat @ fn, x_flat[k] = x[k // D, k % D]                        (GEMM)
3. z_c = hc_scale[g(c)] * (r * m_c) + bias_c, g = pre | post | comb group
4. pre = sigmoid(z[0:n]); post = sigmoid(z[n:2n])                       (gates)
5. comb = Sinkhorn_R(exp(Z)), Z[i, j] = z[2n + i*n + j]                 (mixing)
6. y[d] = sum_i pre_i * x[i, d]                                         (reduce)

Readings (the pages give no formulas; each choice is the plainest one the
calls on the pages support, and is marked "Reading:" where it is applied):
fn rows are stream-major (residual memory order); fn columns are
[pre | post | comb row-major]; the RMS is over all n*D elements with eps inside
the root and scales the GEMM output; the bias is added after hc_scale and is
not RMS-scaled; both gates are the plain logistic function; Sinkhorn makes the
logits positive with exp (after an exact per-row max shift), and one repeat is
a row normalisation followed by a column normalisation, so the last step
always normalises columns; comb[i, j] weighs input stream i into output
stream j.

Parity status: pre_logits, gates, sinkhorn, mhc_pre, mhc_post,
mhc_post_combine_norm and mhc_post_pre are pinned by tests/test_oracle_pins.py (closed forms,
invariants, exact rational arithmetic, brute force, library routines).
The conventions listed above are readings; the pins check their
self-consistency, not the pages.
"""

from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# Storage formats.  bf16 tensors travel as numpy uint16 bit patterns; f32
# tensors as float32.  Decoding is exact; encoding rounds to nearest even.
# --------------------------------------------------------------------------


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):   # NaN payloads widen to NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_f32(x) -> np.ndarray:
    """float64 -> float32, round to nearest even (IEEE default)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f64_to_bf16_bits(x) -> np.ndarray:
    """float64 -> float32 -> bfloat16, each step round-to-nearest-even.

    Reading: outputs stored as bf16 are produced by an fp32 datapath, so the
    oracle rounds to fp32 first; a double-rounding difference from rounding
    float64 straight to bf16 is at most one bf16 unit in the last place.
    NaN stays NaN (quiet); overflow past the largest bf16 becomes infinity.
    """
    f = np.ascontiguousarray(f64_to_f32(x))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    out = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x0040)).astype(np.uint16)
    return out


def decode(a, dtype: str) -> np.ndarray:
    """Stored tensor (``'bf16'`` bits or ``'f32'``) -> float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def encode(x, dtype: str) -> np.ndarray:
    """float64 -> stored tensor in ``dtype`` (round to nearest even)."""
    if dtype == "bf16":
        return f64_to_bf16_bits(x)
    if dtype == "f32":
        return f64_to_f32(x)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# mhc_pre, step by step.
# --------------------------------------------------------------------------


def logit_groups(n: int) -> np.ndarray:
    """Group index of each of the n(n+2) logits: 0 = pre, 1 = post, 2 = comb.

    Reading: fn's columns are ordered [pre_0..pre_{n-1} | post_0..post_{n-1} |
    comb row-major (i, j)], and hc_scale holds one factor per group, in that
    order ([P1] section 2 passes hc_scale as one tensor beside fn).
    """
    g = np.empty(n * (n + 2), dtype=np.int64)
    g[:n] = 0
    g[n:2 * n] = 1
    g[2 * n:] = 2
    return g


def pre_logits(x, fn, hc_scale, bias, eps: float):
    """RMS factor, mixing GEMM, hc_scale and bias for a block of tokens.

    x: float64 [T, n, D]; fn: [n*D, n(n+2)]; hc_scale: [3]; bias: [n(n+2)].
    Returns (z, r, m, s): logits [T, N], RMS factor [T], GEMM output [T, N],
    sum of squares [T], all float64.

    [P1] section 3 names the pre GEMM "gemm_sqrsum": the per-token sum of
    squares is taken over the same row the GEMM contracts.
    Reading: the RMS runs over all n*D elements of the token with eps inside
    the root; scaling the GEMM output by r equals normalising x first because
    the GEMM is linear; z = hc_scale[group] * (r * m) + bias.
    """
    x = np.asarray(x, dtype=np.float64)
    T, n, D = x.shape
    K = n * D
    fn = np.asarray(fn, dtype=np.float64)
    if fn.shape != (K, n * (n + 2)):
        raise ValueError(f"fn has shape {fn.shape}, expected {(K, n * (n + 2))}")
    # Reading: row k of fn multiplies x[k // D, k % D] (stream-major, the
    # residual's own memory order).
    xf = x.reshape(T, K)
    s = np.sum(xf * xf, axis=1)
    r = 1.0 / np.sqrt(s / K + eps)
    m = xf @ fn
    alpha = np.asarray(hc_scale, dtype=np.float64)[logit_groups(n)]
    z = alpha[None, :] * (r[:, None] * m) + np.asarray(bias, dtype=np.float64)[None, :]
    return z, r, m, s


def sigmoid(u) -> np.ndarray:
    """Logistic function 1 / (1 + e^-u) in float64."""
    u = np.asarray(u, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-u))


def gates(z, n: int):
    """pre and post gates from the logits z [T, n(n+2)].

    Reading: both gates are the plain logistic function of their logits, with
    no extra scale or offset; post is the fp32 [T, n] tensor that [P1]
    section 2 squeezes from [T, n, 1].
    """
    z = np.asarray(z, dtype=np.float64)
    return sigmoid(z[:, :n]), sigmoid(z[:, n:2 * n])


def sinkhorn(Z, repeat: int) -> np.ndarray:
    """Sinkhorn normalisation of comb logits Z [T, n, n] -> comb [T, n, n].

    [P1] closing list: the fused kernel runs the Sinkhorn iterations; [P1]
    section 2 passes their count as sinkhorn_repeat.
    Reading: entries are made positive with exp after subtracting each row's
    maximum (exact: the first row normalisation removes any per-row factor);
    one repeat is a row normalisation (each row sums to 1) followed by a
    column normalisation (each column sums to 1); no epsilon is added.
    """
    if repeat < 1:
        raise ValueError("sinkhorn repeat must be >= 1")
    Z = np.asarray(Z, dtype=np.float64)
    M = np.exp(Z - Z.max(axis=2, keepdims=True))
    for _ in range(repeat):
        M = M / M.sum(axis=2, keepdims=True)   # rows i: sum over j is 1
        M = M / M.sum(axis=1, keepdims=True)   # columns j: sum over i is 1
    return M


def stream_reduce(pre, x) -> np.ndarray:
    """y[t, d] = sum_i pre[t, i] * x[t, i, d] in float64.

    [P1] section 2: y is the [T, D] input of the block, one row per token.
    Reading: the streams are weighted by the pre gate and summed, with no
    normalisation of the weights.
    """
    return np.einsum("ti,tid->td", pre, x)


def _check_tokens(a, T, shape_tail, name):
    a = np.asarray(a)
    if a.shape != (T,) + tuple(shape_tail):
        raise ValueError(f"{name} has shape {a.shape}, expected {(T,) + tuple(shape_tail)}")
    return a


def mhc_pre(residual, fn, hc_scale, bias, *, n: int, D: int, dtype: str,
            sinkhorn_repeat: int, eps: float, chunk: int = 1024,
            intermediates: bool = False):
    """mhc_pre: residual [T, n, D] -> (post [T, n] f32, comb [T, n, n] f32, y [T, D]).

    [P1] section 2: the pre call takes the residual, fn, hc_scale and the
    Sinkhorn repeat count and returns post, comb and y, in that order.
    y is stored in the residual's dtype; post and comb in fp32.
    Reading: y[d] = sum_i pre_i * x[i, d] (the streams weighted by the pre
    gate, not normalised); the result is rounded once from float64.
    Tokens are independent, so the oracle works through them ``chunk`` at a
    time to bound memory; this is not a reordering of any sum.

    With ``intermediates=True`` also returns a dict of float64 arrays
    (s, r, m, z, pre, post, comb, y) before storage rounding.
    """
    T = np.asarray(residual).shape[0]
    residual = _check_tokens(residual, T, (n, D), "residual")
    N = n * (n + 2)
    post_out = np.empty((T, n), dtype=np.float32)
    comb_out = np.empty((T, n, n), dtype=np.float32)
    y_out = np.empty((T, D), dtype=np.uint16 if dtype == "bf16" else np.float32)
    inter = {k: [] for k in ("s", "r", "m", "z", "pre", "post", "comb", "y")} if intermediates else None
    for t0 in range(0, T, chunk):
        x = decode(residual[t0:t0 + chunk], dtype)
        z, r, m, s = pre_logits(x, fn, hc_scale, bias, eps)
        pre, post = gates(z, n)
        comb = sinkhorn(z[:, 2 * n:].reshape(-1, n, n), sinkhorn_repeat)
        y = stream_reduce(pre, x)
        post_out[t0:t0 + chunk] = f64_to_f32(post)
        comb_out[t0:t0 + chunk] = f64_to_f32(comb)
        y_out[t0:t0 + chunk] = encode(y, dtype)
        if inter is not None:
            for k, v in (("s", s), ("r", r), ("m", m), ("z", z), ("pre", pre),
                         ("post", post), ("comb", comb), ("y", y)):
                inter[k].append(v)
    assert N == np.asarray(fn).shape[1]
    if inter is not None:
        empty = {"s": (0,), "r": (0,), "m": (0, N), "z": (0, N), "pre": (0, n),
                 "post": (0, n), "comb": (0, n, n), "y": (0, D)}
        inter = {k: (np.concatenate(v) if v else np.zeros(empty[k])) for k, v in inter.items()}
        return post_out, comb_out, y_out, inter
    return post_out, comb_out, y_out


# --------------------------------------------------------------------------
# mhc_post and the fused post + combine + RMSNorm.
# --------------------------------------------------------------------------


def post_mix(h, x, post, comb) -> np.ndarray:
    """out[t, j, d] = post[t, j] * h[t, d] + sum_i comb[t, i, j] * x[t, i, d], float64.

    [P1] section 2: the post call mixes the block output with the residual
    streams using post and comb, writing a tensor shaped like the residual.
    Reading: comb[i, j] weighs input stream i into output stream j.
    """
    return post[:, :, None] * h[:, None, :] + np.einsum("tij,tid->tjd", comb, x)


def mhc_post(h, residual, post, comb, *, n: int, D: int, dtype: str, chunk: int = 1024):
    """mhc_post: out [T, n, D] in the residual's dtype, rounded once.

    post [T, n] and comb [T, n, n] are taken as stored (fp32) and widened
    exactly; h [T, D] and residual [T, n, D] are in ``dtype``.
    """
    T = np.asarray(residual).shape[0]
    residual = _check_tokens(residual, T, (n, D), "residual")
    h = _check_tokens(h, T, (D,), "h")
    post = _check_tokens(np.asarray(post, dtype=np.float32), T, (n,), "post")
    comb = _check_tokens(np.asarray(comb, dtype=np.float32), T, (n, n), "comb")
    out = np.empty((T, n, D), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for t0 in range(0, T, chunk):
        sl = slice(t0, t0 + chunk)
        o = post_mix(decode(h[sl], dtype), decode(residual[sl], dtype),
                     post[sl].astype(np.float64), comb[sl].astype(np.float64))
        out[sl] = encode(o, dtype)
    return out


def rms_norm(c, weight, eps: float) -> np.ndarray:
    """(c * (mean(c^2) + eps)^-1/2) * weight over the last axis, float64.

    [P2] section 1: the combined row is RMS-normalised before it is stored.
    Reading: mean over D, eps inside the root, the weight applied after the
    scaling.
    """
    c = np.asarray(c, dtype=np.float64)
    q = 1.0 / np.sqrt(np.mean(c * c, axis=-1, keepdims=True) + eps)
    return (c * q) * np.asarray(weight, dtype=np.float64)


def combine_intermediates(h, x, post, comb, w, dtype: str):
    """The fused tail's stored intermediates (o [T, n, D], c [T, D]) as float64.

    [P2] section 1: the post rows and the combined row are bf16 intermediates
    (the ``collapsed`` row is a bf16 buffer).
    Reading: each post row o_j is exactly what ``mhc_post`` stores (the
    float64 post mix rounded once to the storage type); the combined row is
    c = sum_j w_j * o_j, formed in float64 from those stored rows and rounded
    once to the storage type.
    """
    hv = decode(h, dtype)
    xv = decode(x, dtype)
    o = decode(encode(post_mix(hv, xv, np.asarray(post, dtype=np.float32).astype(np.float64),
                               np.asarray(comb, dtype=np.float32).astype(np.float64)), dtype), dtype)
    c = np.einsum("tj,tjd->td", np.asarray(w, dtype=np.float32).astype(np.float64), o)
    return o, decode(encode(c, dtype), dtype)


def mhc_post_combine_norm(h, residual, post, comb, combine_w, norm_weight, *,
                          n: int, D: int, dtype: str, norm_eps: float, chunk: int = 1024):
    """Fused post mix + next-layer combine + RMSNorm -> (normalized [T, D], out [T, n, D]).

    [P2] section 1: one row at a time, the post result is combined across the
    n streams into a bf16 ``collapsed`` row of D values, which is then
    RMS-normalised; [P2] section 2 stores it as ``normalized``.
    Reading: out_j is the post result rounded to the residual dtype (the
    same value ``mhc_post`` stores) and c is the combined row rounded to the
    residual dtype, both formed in float64 as ``combine_intermediates``
    states; the RMSNorm runs in float64 on that rounded c and is rounded once.
    combine_w [T, n] and norm_weight [D] are fp32.
    """
    T = np.asarray(residual).shape[0]
    residual = _check_tokens(residual, T, (n, D), "residual")
    h = _check_tokens(h, T, (D,), "h")
    w = _check_tokens(np.asarray(combine_w, dtype=np.float32), T, (n,), "combine_w")
    g = np.asarray(norm_weight, dtype=np.float32)
    if g.shape != (D,):
        raise ValueError(f"norm_weight has shape {g.shape}, expected {(D,)}")
    post = _check_tokens(np.asarray(post, dtype=np.float32), T, (n,), "post")
    comb = _check_tokens(np.asarray(comb, dtype=np.float32), T, (n, n), "comb")
    odt = np.uint16 if dtype == "bf16" else np.float32
    out = np.empty((T, n, D), dtype=odt)
    normalized = np.empty((T, D), dtype=odt)
    for t0 in range(0, T, chunk):
        sl = slice(t0, t0 + chunk)
        o, c = combine_intermediates(h[sl], residual[sl], post[sl], comb[sl], w[sl], dtype)
        out[sl] = encode(o, dtype)
        normalized[sl] = encode(rms_norm(c, g.astype(np.float64), norm_eps), dtype)
    return normalized, out


# --------------------------------------------------------------------------
# The layer boundary: mhc_post of the finished layer, then mhc_pre of the next.
# --------------------------------------------------------------------------


def mhc_post_pre(h, residual, post, comb, fn, hc_scale, bias, *, n: int, D: int, dtype: str,
                 sinkhorn_repeat: int, eps: float, chunk: int = 1024):
    """Layer boundary -> (out [T, n, D], post' [T, n] f32, comb' [T, n, n] f32, y' [T, D]).

    [P1] section 2: a layer ends with the post call, whose result (shaped like
    the residual) is the next layer's residual, and the next layer starts with
    the pre call on it. [P2] section 1 fuses the post mix with the next
    layer's input processing; this is the same boundary with the next layer's
    full pre step. The definition is the two calls in sequence: out is
    ``mhc_post`` rounded to the residual dtype, and ``mhc_pre`` reads that
    stored value with the next layer's fn, hc_scale and bias.
    """
    out = mhc_post(h, residual, post, comb, n=n, D=D, dtype=dtype, chunk=chunk)
    post_n, comb_n, y_n = mhc_pre(out, fn, hc_scale, bias, n=n, D=D, dtype=dtype,
                                  sinkhorn_repeat=sinkhorn_repeat, eps=eps, chunk=chunk)
    return out, post_n, comb_n, y_n
