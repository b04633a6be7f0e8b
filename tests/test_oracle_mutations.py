"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each one."""

import numpy as np
import pytest

import oracle.mhc_oracle as O
from oracle_pins import ALL_PINS

_orig = {k: getattr(O, k) for k in ("pre_logits", "gates", "sinkhorn", "post_mix", "stream_reduce",
                                    "rms_norm", "f64_to_bf16_bits", "logit_groups", "mhc_post_combine_norm",
                                    "combine_intermediates", "mhc_post_pre", "mhc_pre", "mhc_post", "encode")}


def _sinkhorn_cols_first(Z, repeat):
    M = np.exp(Z - Z.max(axis=2, keepdims=True))
    for _ in range(repeat):
        M = M / M.sum(axis=1, keepdims=True)
        M = M / M.sum(axis=2, keepdims=True)
    return M


def _sinkhorn_half_steps(Z, repeat):
    M = np.exp(Z - Z.max(axis=2, keepdims=True))
    for s in range(repeat):
        M = M / M.sum(axis=2 if s % 2 == 0 else 1, keepdims=True)
    return M


def _sinkhorn_transposed(Z, repeat):
    return _orig["sinkhorn"](Z, repeat).transpose(0, 2, 1)


def _sinkhorn_softmax_only(Z, repeat):
    M = np.exp(Z - Z.max(axis=2, keepdims=True))
    return M / M.sum(axis=2, keepdims=True)


def _pre_logits_with(x, fn, hc_scale, bias, eps, rms):
    x = np.asarray(x, dtype=np.float64)
    T, n, D = x.shape
    xf = x.reshape(T, n * D)
    s = np.sum(xf * xf, axis=1)
    r = rms(s, n, D, eps)
    m = xf @ np.asarray(fn, dtype=np.float64)
    alpha = np.asarray(hc_scale, dtype=np.float64)[_orig["logit_groups"](n)]
    return alpha[None, :] * (r[:, None] * m) + np.asarray(bias)[None, :], r, m, s


def _pre_logits_eps_outside(x, fn, hc_scale, bias, eps):
    return _pre_logits_with(x, fn, hc_scale, bias, eps, lambda s, n, D, e: 1.0 / np.sqrt(s / (n * D)) + e)


def _pre_logits_mean_over_d(x, fn, hc_scale, bias, eps):
    return _pre_logits_with(x, fn, hc_scale, bias, eps, lambda s, n, D, e: 1.0 / np.sqrt(s / D + e))


def _pre_logits_d_major(x, fn, hc_scale, bias, eps):
    x = np.asarray(x, dtype=np.float64)
    T, n, D = x.shape
    return _orig["pre_logits"](np.ascontiguousarray(x.transpose(0, 2, 1)).reshape(T, n, D), fn, hc_scale, bias, eps)


def _pre_logits_bias_scaled(x, fn, hc_scale, bias, eps):
    n = np.asarray(x).shape[1]
    alpha = np.asarray(hc_scale, dtype=np.float64)[_orig["logit_groups"](n)]
    return _orig["pre_logits"](x, fn, hc_scale, np.asarray(bias) * alpha, eps)


def _groups_swapped(n):
    g = _orig["logit_groups"](n)
    return np.where(g == 1, 2, np.where(g == 2, 1, g))


def _gates_sign(z, n):
    pre, post = _orig["gates"](-np.asarray(z), n)
    return pre, post


def _gates_swapped(z, n):
    pre, post = _orig["gates"](z, n)
    return post, pre


def _post_mix_transposed(h, x, post, comb):
    return _orig["post_mix"](h, x, post, np.swapaxes(comb, 1, 2))


def _post_mix_no_h(h, x, post, comb):
    return _orig["post_mix"](np.zeros_like(h), x, post, comb)


def _reduce_mean(pre, x):
    return _orig["stream_reduce"](pre, x) / pre.shape[1]


def _reduce_normalised(pre, x):
    return _orig["stream_reduce"](pre / pre.sum(axis=1, keepdims=True), x)


def _rms_eps_outside(c, weight, eps):
    c = np.asarray(c, dtype=np.float64)
    q = 1.0 / np.sqrt(np.mean(c * c, axis=-1, keepdims=True)) + eps
    return (c * q) * np.asarray(weight, dtype=np.float64)


def _bf16_truncate(x):
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _combine_c_unrounded(h, x, post, comb, w, dtype):
    o, c = _orig["combine_intermediates"](h, x, post, comb, w, dtype)
    return o, np.einsum("tj,tjd->td", np.asarray(w, dtype=np.float64), o)


def _combine_weights_reversed(h, x, post, comb, w, dtype):
    return _orig["combine_intermediates"](h, x, post, comb, np.asarray(w)[:, ::-1], dtype)


def _boundary_pre_on_old_residual(h, residual, post, comb, fn, hc_scale, bias, *, n, D, dtype, sinkhorn_repeat,
                                  eps, chunk=1024):
    out = _orig["mhc_post"](h, residual, post, comb, n=n, D=D, dtype=dtype)
    return (out,) + _orig["mhc_pre"](residual, fn, hc_scale, bias, n=n, D=D, dtype=dtype,
                                     sinkhorn_repeat=sinkhorn_repeat, eps=eps)


def _boundary_pre_on_unrounded(h, residual, post, comb, fn, hc_scale, bias, *, n, D, dtype, sinkhorn_repeat,
                               eps, chunk=1024):
    out = _orig["mhc_post"](h, residual, post, comb, n=n, D=D, dtype=dtype)
    mix = O.post_mix(O.decode(h, dtype), O.decode(residual, dtype), np.asarray(post, np.float64),
                     np.asarray(comb, np.float64)).astype(np.float32)
    pn, cn, yn = _orig["mhc_pre"](mix, fn, hc_scale, bias, n=n, D=D, dtype="f32", sinkhorn_repeat=sinkhorn_repeat,
                                  eps=eps)
    return out, pn, cn, _orig["encode"](yn.astype(np.float64), dtype)


MUTATIONS = {
    "boundary pre reads the finished layer's residual": ("mhc_post_pre", _boundary_pre_on_old_residual),
    "boundary pre reads the post mix before storage rounding": ("mhc_post_pre", _boundary_pre_on_unrounded),
    "combined row kept unrounded": ("combine_intermediates", _combine_c_unrounded),
    "combine weights applied to the wrong streams": ("combine_intermediates", _combine_weights_reversed),
    "sinkhorn columns first": ("sinkhorn", _sinkhorn_cols_first),
    "sinkhorn repeat counts half steps": ("sinkhorn", _sinkhorn_half_steps),
    "sinkhorn output transposed": ("sinkhorn", _sinkhorn_transposed),
    "sinkhorn stops after a row softmax": ("sinkhorn", _sinkhorn_softmax_only),
    "rms eps outside the root": ("pre_logits", _pre_logits_eps_outside),
    "rms mean over D instead of n*D": ("pre_logits", _pre_logits_mean_over_d),
    "fn rows taken d-major": ("pre_logits", _pre_logits_d_major),
    "bias scaled by hc_scale": ("pre_logits", _pre_logits_bias_scaled),
    "hc_scale post/comb groups swapped": ("logit_groups", _groups_swapped),
    "gate sign flipped": ("gates", _gates_sign),
    "pre and post gates swapped": ("gates", _gates_swapped),
    "post mix reads comb transposed": ("post_mix", _post_mix_transposed),
    "post mix drops post*h": ("post_mix", _post_mix_no_h),
    "stream reduce averages": ("stream_reduce", _reduce_mean),
    "stream reduce normalises pre": ("stream_reduce", _reduce_normalised),
    "rmsnorm eps outside the root": ("rms_norm", _rms_eps_outside),
    "bf16 rounding truncates": ("f64_to_bf16_bits", _bf16_truncate),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(O, attr, bad)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(O)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake: {name}"
