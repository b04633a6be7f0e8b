"""Seeded synthetic inputs for mHC pre/post mixing.

This module only draws random inputs in the shapes, dtypes and value
distributions of the workloads; it holds none of the mixing arithmetic. Both
the CPU oracle (through the tests) and the HIP path consume its arrays, so the
two sides see bit-identical inputs.

Workloads (DeepSeek-V4-style layers with n = 4 residual streams; the pages
describe prefill at hidden sizes n*D of 16384 and 28672, and decode
verification batches at concurrency 32/64 with D = 5120):

==================== ======== === ===== ===== ==========================================
name                 T        n   D     dtype notes
==================== ======== === ===== ===== ==========================================
tiny-f32             8        4   256   f32   fn ~ N(0, 0.02)
prefill-d4096        2048     4   4096  bf16  fn ~ N(0, 0.01); one split (n_splits = 1)
prefill-d7168        2048     4   7168  bf16  fn ~ N(0, 0.01); the throughput workload
decode-t32-d5120     32       4   5120  bf16  fused post + combine + RMSNorm
decode-t64-d5120     64       4   5120  bf16  fused post + combine + RMSNorm
prefill-t16384-d7168 16384    4   7168  bf16  1 % outliers x50; split-K (n_splits > 1)
==================== ======== === ===== ===== ==========================================

Distributions: residual ~ N(0, residual_std) (1 in every named workload) and
h ~ N(0, 1); fn ~ N(0, fn_std) (the second number is the standard deviation);
bias ~ N(0, 0.1); hc_scale = (1, 1, 1) in every named workload (other values,
like other repeat counts and eps, are parity cases of the knobs);
combine_w ~ U(0, 1); norm_weight ~ U(0.5, 1.5). The outlier workload multiplies
each residual element by 50 with probability 0.01 (a Bernoulli mask) before
rounding. Values are drawn in float32 and rounded to bf16 to nearest even.

Every array has its own random stream, spawned from the workload's seed, so
arrays can be drawn in any order and in chunks without changing any value.
"""

from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

# stream ids spawned from the workload seed
_S_RESIDUAL, _S_FN, _S_BIAS, _S_H, _S_OUTLIER, _S_COMBINE_W, _S_NORM_W, _S_NEXT_FN, _S_MIX = range(9)
_N_STREAMS = 9
_CHUNK_TOKENS = 256


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape, dtype, value distribution and call knobs of one workload."""
    name: str
    T: int
    n: int
    D: int
    dtype: str                 # "bf16" or "f32": dtype of residual, h, y, out
    seed: int
    fn_std: float = 0.01
    bias_std: float = 0.1
    outlier_p: float = 0.0
    outlier_scale: float = 50.0
    hc_scale: tuple = (1.0, 1.0, 1.0)   # (pre, post, comb) group factors
    residual_std: float = 1.0
    sinkhorn_repeat: int = 20
    eps: float = 1e-6
    norm_eps: float = 1e-6
    n_splits: int = 0          # 0 lets the library choose
    combine: bool = False      # fused post + combine + RMSNorm inputs too

    @property
    def K(self) -> int:
        return self.n * self.D

    @property
    def N(self) -> int:
        return self.n * (self.n + 2)


SPECS = {
    s.name: s
    for s in (
        Spec("tiny-f32", T=8, n=4, D=256, dtype="f32", seed=1001, fn_std=0.02, combine=True),
        Spec("prefill-d4096", T=2048, n=4, D=4096, dtype="bf16", seed=1002, n_splits=1),
        Spec("prefill-d7168", T=2048, n=4, D=7168, dtype="bf16", seed=1003),
        Spec("decode-t32-d5120", T=32, n=4, D=5120, dtype="bf16", seed=1004, combine=True),
        Spec("decode-t64-d5120", T=64, n=4, D=5120, dtype="bf16", seed=1014, combine=True),
        Spec("prefill-t16384-d7168", T=16384, n=4, D=7168, dtype="bf16", seed=1005,
             outlier_p=0.01, n_splits=4),
    )
}

THROUGHPUT_WORKLOAD = "prefill-d7168"


def spec(name: str, **overrides) -> Spec:
    """A named workload, optionally with fields replaced (e.g. a smaller T)."""
    return dataclasses.replace(SPECS[name], **overrides) if overrides else SPECS[name]


def custom(T: int, n: int, D: int, dtype: str = "bf16", seed: int = 7, **kw) -> Spec:
    """An ad-hoc workload (parity sweeps, edge cases) with the default distributions."""
    return Spec(f"custom-T{T}-n{n}-D{D}-{dtype}-s{seed}", T=T, n=n, D=D, dtype=dtype, seed=seed, **kw)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest even); returns uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("generator produced a non-finite value")
    u = a.view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


@dataclasses.dataclass
class Inputs:
    """Host arrays of one workload. bf16 arrays are uint16 bit patterns."""
    spec: Spec
    residual: np.ndarray              # [T, n, D]
    fn: np.ndarray                    # [n*D, n(n+2)] float32
    hc_scale: np.ndarray              # [3] float32
    bias: np.ndarray                  # [n(n+2)] float32
    h: np.ndarray                     # [T, D]
    combine_w: Optional[np.ndarray]   # [T, n] float32
    norm_weight: Optional[np.ndarray]  # [D] float32

    def arrays(self):
        out = {"residual": self.residual, "fn": self.fn, "hc_scale": self.hc_scale,
               "bias": self.bias, "h": self.h}
        if self.combine_w is not None:
            out["combine_w"] = self.combine_w
            out["norm_weight"] = self.norm_weight
        return out

    def checksums(self) -> dict:
        """SHA-256 of every array's bytes (recorded beside measurements)."""
        return {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()
                for k, v in self.arrays().items()}


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else np.ascontiguousarray(a32, dtype=np.float32)


def _token_tensor(rng, T: int, tail: tuple, dtype: str, outlier_rng=None, p=0.0, scale=1.0, std=1.0):
    """N(0, std) tensor [T, *tail] drawn in fixed token chunks, optionally with outliers."""
    out = np.empty((T,) + tail, dtype=np.uint16 if dtype == "bf16" else np.float32)
    for t0 in range(0, T, _CHUNK_TOKENS):
        t1 = min(T, t0 + _CHUNK_TOKENS)
        a = rng.standard_normal((t1 - t0,) + tail, dtype=np.float32)
        if std != 1.0:
            a = a * np.float32(std)
        if outlier_rng is not None and p > 0.0:
            mask = outlier_rng.random((t1 - t0,) + tail, dtype=np.float32) < np.float32(p)
            a = np.where(mask, a * np.float32(scale), a)
        out[t0:t1] = _store(a, dtype)
    return out


def generate(s: Spec) -> Inputs:
    """Draw every input array of workload ``s`` (deterministic in ``s``)."""
    rngs = [np.random.default_rng(c) for c in np.random.SeedSequence(s.seed).spawn(_N_STREAMS)]
    residual = _token_tensor(rngs[_S_RESIDUAL], s.T, (s.n, s.D), s.dtype,
                             rngs[_S_OUTLIER] if s.outlier_p > 0 else None, s.outlier_p, s.outlier_scale,
                             s.residual_std)
    fn = (rngs[_S_FN].standard_normal((s.K, s.N), dtype=np.float32) * np.float32(s.fn_std)).astype(np.float32)
    bias = (rngs[_S_BIAS].standard_normal((s.N,), dtype=np.float32) * np.float32(s.bias_std)).astype(np.float32)
    h = _token_tensor(rngs[_S_H], s.T, (s.D,), s.dtype)
    hc_scale = np.asarray(s.hc_scale, dtype=np.float32)
    combine_w = norm_weight = None
    if s.combine:
        combine_w = rngs[_S_COMBINE_W].random((s.T, s.n), dtype=np.float32)
        norm_weight = (np.float32(0.5) + rngs[_S_NORM_W].random((s.D,), dtype=np.float32)).astype(np.float32)
    return Inputs(s, residual, fn, hc_scale, bias, h, combine_w, norm_weight)


def next_layer_fn(s: Spec) -> np.ndarray:
    """fn of the next layer for the layer-boundary call: the same distribution as ``fn``, its own stream."""
    rng = np.random.default_rng(np.random.SeedSequence(s.seed).spawn(_N_STREAMS)[_S_NEXT_FN])
    return (rng.standard_normal((s.K, s.N), dtype=np.float32) * np.float32(s.fn_std)).astype(np.float32)


def mixing_weights(s: Spec):
    """post [T, n] ~ U(0, 1) and comb [T, n, n] ~ U(0, 1) / n (float32) for post-step tests at sizes where
    computing them with a pre step on the host would be slow; drawn directly, not by the method."""
    rng = np.random.default_rng(np.random.SeedSequence(s.seed).spawn(_N_STREAMS)[_S_MIX])
    post = rng.random((s.T, s.n), dtype=np.float32)
    comb = (rng.random((s.T, s.n, s.n), dtype=np.float32) / np.float32(s.n)).astype(np.float32)
    return post, comb
