"""mHC (multi-stream hyper-connection) pre/post mixing for MI355X (gfx950).

A thin Python binding over the C ABI of ``libmhc.so`` (declared in
``include/mhc.h``). Every step of the computation runs in the library's HIP
kernels; this module only checks tensor metadata, allocates outputs with torch
when the caller does not pass them (and a workspace, kept per device and
launch stream for later calls), and marshals pointers and the current HIP
stream. There is no CPU fallback: if the library
is not built, every call raises.

Functions mirror the C entry points: ``mhc_pre``, ``mhc_post``,
``mhc_post_combine_norm``, ``mhc_post_pre`` (the layer boundary: post, then
the next layer's pre), ``mhc_pre_workspace_bytes``, ``mhc_pre_splits``,
``mhc_post_pre_fused``. With ``prepare=True`` the four compute wrappers check
and marshal once and return a ``PreparedCall`` that repeats the call.
"""

from __future__ import annotations

import contextlib
import ctypes
import os

__all__ = [
    "MhcError", "lib", "library_path", "mhc_pre", "mhc_post", "mhc_post_combine_norm",
    "mhc_pre_workspace_bytes", "mhc_pre_splits", "mhc_pre_sync_timeouts", "mhc_post_pre", "mhc_post_pre_fused",
    "mhc_pre_static", "mhc_pre_plan_info", "MHC_PRE_STATIC_SCRATCH_BYTES", "MHC_BF16", "MHC_F32", "PreparedCall",
    "release_workspaces",
]

MHC_BF16 = 0
MHC_F32 = 1
MHC_PRE_STATIC_SCRATCH_BYTES = 32 << 20   # the library's per-GPU scratch for mhc_pre_static

_LIB = None


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmhc.so")


class MhcError(RuntimeError):
    """A negative status returned by the C ABI."""

    def __init__(self, fn: str, status: int):
        L = lib()
        msg = L.mhc_status_string(status).decode()
        if status == -5:
            msg += f" ({L.mhc_last_error().decode()})"
        super().__init__(f"{fn}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load ``libmhc.so`` (once) and declare the C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m mhc_hyper_connection_pre_amd.build` "
                           "(there is no CPU fallback)")
    _LIB = load_library(path)
    return _LIB


def load_library(path: str) -> ctypes.CDLL:
    """Load a build of the C ABI at `path` and declare its signatures (``lib()`` loads the in-tree one)."""
    L = ctypes.CDLL(path)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.mhc_status_string.argtypes = [I]
    L.mhc_status_string.restype = ctypes.c_char_p
    L.mhc_last_error.argtypes = []
    L.mhc_last_error.restype = ctypes.c_char_p
    L.mhc_pre_splits.argtypes = [I64, I, I64, I, I]
    L.mhc_pre_splits.restype = I
    L.mhc_pre_workspace_bytes.argtypes = [I64, I, I64, I, I]
    L.mhc_pre_workspace_bytes.restype = SZ
    L.mhc_pre_sync_timeouts.argtypes = [P, SZ, I64, I, I64, I, I, P]
    L.mhc_pre_sync_timeouts.restype = I
    L.mhc_pre.argtypes = [P, P, P, P, I, P, P, P, I64, I, I64, I, F, I, P, SZ, P]
    L.mhc_pre.restype = I
    L.mhc_pre_static.argtypes = [P, P, P, P, I, P, P, P, I64, I, I64, I, F, I, P]
    L.mhc_pre_static.restype = I
    L.mhc_post.argtypes = [P, P, P, P, P, I, I64, I, I64, P]
    L.mhc_post.restype = I
    L.mhc_post_combine_norm.argtypes = [P, P, P, P, P, P, P, P, F, I, I64, I, I64, P]
    L.mhc_post_combine_norm.restype = I
    L.mhc_post_pre.argtypes = [P, P, P, P, P, P, P, P, I, P, P, P, I64, I, I64, I, F, I, P, SZ, P]
    L.mhc_post_pre.restype = I
    L.mhc_post_pre_fused.argtypes = [I64, I, I64, I, I]
    L.mhc_post_pre_fused.restype = I
    L.mhc_pre_plan_info.argtypes = [I64, I, I64, I, I, I, ctypes.POINTER(I)]
    L.mhc_pre_plan_info.restype = I
    return L


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MHC_BF16
    if t.dtype == torch.float32:
        return MHC_F32
    raise TypeError(f"residual-shaped tensors must be bfloat16 or float32, got {t.dtype}")


def _ptr(t) -> int:
    return t.data_ptr() if t is not None else None


def _check(t, shape, dtype, device, name):
    # one cheap test for the usual case (a decode step spends microseconds here)
    if t is not None and t.shape == shape and t.dtype == dtype and t.device == device and t.is_contiguous():
        return
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    raise ValueError(f"{name} must be contiguous")


def _gpu_device(t, name):
    """The device of ``t``, which must be a GPU tensor (the kernels dereference its address on the GPU)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} is on {t.device}; the kernels need tensors on a GPU")
    return t.device


def _workspace_bytes(ws, device) -> int:
    """Size in bytes of a caller's workspace tensor, after checking that the kernels can use it."""
    if ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, expected {device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return ws.numel() * ws.element_size()


def _on(stream):
    """Allocate (and zero) on the launch stream: the caching allocator then orders any later reuse of the
    memory after the kernels, and the zeroing runs before them on the same stream."""
    return _torch().cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _stream(device, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


# Workspaces this binding keeps for calls that pass none, one per (device, launch stream). The
# single-pass kernels carry their state from call to call in the workspace (the last epoch and a
# shape marker; a call of another shape, or of the two-pass path, re-arms it on the GPU), so the
# zeroing of its status words at allocation serves every later call and such a call is one
# launch, not a fill and a launch. Calls on one stream run in order and can share it; calls on
# another stream get their own. A call made while the current stream is being captured into a
# graph allocates a fresh workspace, as before (a graph replays with the memory it captured).
_WORKSPACES: dict = {}


def _default_workspace(L, T, n, D, n_splits, dt, dev, stream):
    torch = _torch()
    need = max(L.mhc_pre_workspace_bytes(T, n, D, n_splits, dt), 256)
    if torch.cuda.is_current_stream_capturing():
        with _on(stream):
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            ws[:256].zero_()
        return ws
    key = (dev.index, _stream(dev, stream))
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < need:
        # allocated and cleared on the launch stream: a smaller one it replaces returns to that
        # stream's pool, which hands it out again only after the calls queued there
        with _on(stream):
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            ws[:256].zero_()
        _WORKSPACES[key] = ws
    return ws


def release_workspaces() -> None:
    """Drop the workspaces kept for calls that pass none (the memory returns to torch's allocator)."""
    _WORKSPACES.clear()


class PreparedCall:
    """One library call with its tensors checked and its C arguments marshalled once.

    Each call of the object launches the entry point again with the same
    arguments and returns the same output tensors; the library still checks
    the arguments and plans the launch on every call. For launch loops
    (decode steps) where the per-call checks of this binding would cost more
    host time than the kernels take. The tensors (held here, so their memory
    stays allocated) must keep their storage: an in-place resize or a swapped
    storage leaves stale pointers.
    """

    def __init__(self, name, cfn, args, outputs, keep):
        self.name, self._fn, self._args, self.outputs, self._keep = name, cfn, args, outputs, keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            raise MhcError(self.name, st)
        return self.outputs


def _finish(name, cfn, args, outputs, prepare, keep):
    if prepare:
        return PreparedCall(name, cfn, args, outputs, keep)
    st = cfn(*args)
    if st != 0:
        raise MhcError(name, st)
    return outputs


def mhc_pre_splits(T: int, n: int, D: int, n_splits: int = 0, dtype_code: int = MHC_BF16) -> int:
    st = lib().mhc_pre_splits(T, n, D, n_splits, dtype_code)
    if st < 0:
        raise MhcError("mhc_pre_splits", st)
    return st


def mhc_pre_plan_info(T: int, n: int, D: int, n_splits: int = 0, dtype_code: int = MHC_BF16,
                      boundary: bool = False) -> dict:
    """The plan a call with these sizes takes (``include/mhc.h``: mhc_pre_plan_info)."""
    info = (ctypes.c_int * 5)()
    st = lib().mhc_pre_plan_info(T, n, D, n_splits, dtype_code, 1 if boundary else 0, info)
    if st != 0:
        raise MhcError("mhc_pre_plan_info", st)
    return {"single_pass": bool(info[0]), "splits": info[1], "cols_per_slice": info[2], "generations": info[3],
            "per_wave": info[4] == 1 if info[0] else None}


def mhc_pre_workspace_bytes(T: int, n: int, D: int, n_splits: int = 0, dtype_code: int = MHC_BF16) -> int:
    return lib().mhc_pre_workspace_bytes(T, n, D, n_splits, dtype_code)


def mhc_pre_sync_timeouts(workspace, residual, n_splits: int = 0, stream=None) -> int:
    """Poll timeouts the last mhc_pre on ``workspace`` (for ``residual``'s shape) recorded. Blocks the host."""
    T, n, D = residual.shape
    dev = _gpu_device(residual, "residual")
    st = lib().mhc_pre_sync_timeouts(_ptr(workspace), _workspace_bytes(workspace, dev), T, n, D, n_splits,
                                     _dtype_code(residual), _stream(dev, stream))
    if st < 0:
        raise MhcError("mhc_pre_sync_timeouts", st)
    return st


def mhc_pre(residual, fn, hc_scale, bias, *, sinkhorn_repeat: int = 20, eps: float = 1e-6, n_splits: int = 0,
            post=None, comb=None, y=None, workspace=None, stream=None, prepare: bool = False):
    """post [T, n] f32, comb [T, n, n] f32, y [T, D] = mhc_pre(residual [T, n, D], fn, hc_scale, bias).

    n_splits as in ``include/mhc.h``: 0 = the library's tiling (its tile table, else a heuristic), S > 0 = the
    two-pass path with S split-K partials, -1 = the single-pass kernel, -S = the single-pass kernel with S slices.
    prepare=True returns a ``PreparedCall`` that makes this call when called.
    """
    torch = _torch()
    L = lib()
    T, n, D = residual.shape
    dev = _gpu_device(residual, "residual")
    dt = _dtype_code(residual)
    N = n * (n + 2)
    _check(residual, (T, n, D), residual.dtype, dev, "residual")
    _check(fn, (n * D, N), torch.float32, dev, "fn")
    _check(hc_scale, (3,), torch.float32, dev, "hc_scale")
    _check(bias, (N,), torch.float32, dev, "bias")
    with _on(stream):
        post = torch.empty((T, n), dtype=torch.float32, device=dev) if post is None else post
        comb = torch.empty((T, n, n), dtype=torch.float32, device=dev) if comb is None else comb
        y = torch.empty((T, D), dtype=residual.dtype, device=dev) if y is None else y
    if workspace is None:
        workspace = _default_workspace(L, T, n, D, n_splits, dt, dev, stream)
    _check(post, (T, n), torch.float32, dev, "post")
    _check(comb, (T, n, n), torch.float32, dev, "comb")
    _check(y, (T, D), residual.dtype, dev, "y")
    args = (_ptr(post), _ptr(comb), _ptr(y), _ptr(residual), dt, _ptr(fn), _ptr(hc_scale), _ptr(bias),
            T, n, D, sinkhorn_repeat, eps, n_splits, _ptr(workspace), _workspace_bytes(workspace, dev),
            _stream(dev, stream))
    return _finish("mhc_pre", L.mhc_pre, args, (post, comb, y), prepare, (residual, fn, hc_scale, bias, workspace))


def mhc_pre_static(residual, fn, hc_scale, bias, *, sinkhorn_repeat: int = 20, eps: float = 1e-6,
                   n_splits: int = 0, post=None, comb=None, y=None, stream=None):
    """mhc_pre on the library's own per-GPU scratch (no workspace; the C call allocates nothing).

    For callers that cannot allocate device memory during the call: pass ``post``, ``comb`` and ``y`` (this
    wrapper allocates them with torch only when they are omitted). Sizes whose workspace exceeds
    ``MHC_PRE_STATIC_SCRATCH_BYTES`` raise; calls that overlap on one GPU race on the shared scratch.
    """
    torch = _torch()
    T, n, D = residual.shape
    dev = _gpu_device(residual, "residual")
    dt = _dtype_code(residual)
    N = n * (n + 2)
    _check(residual, (T, n, D), residual.dtype, dev, "residual")
    _check(fn, (n * D, N), torch.float32, dev, "fn")
    _check(hc_scale, (3,), torch.float32, dev, "hc_scale")
    _check(bias, (N,), torch.float32, dev, "bias")
    with _on(stream):
        post = torch.empty((T, n), dtype=torch.float32, device=dev) if post is None else post
        comb = torch.empty((T, n, n), dtype=torch.float32, device=dev) if comb is None else comb
        y = torch.empty((T, D), dtype=residual.dtype, device=dev) if y is None else y
    _check(post, (T, n), torch.float32, dev, "post")
    _check(comb, (T, n, n), torch.float32, dev, "comb")
    _check(y, (T, D), residual.dtype, dev, "y")
    args = (_ptr(post), _ptr(comb), _ptr(y), _ptr(residual), dt, _ptr(fn), _ptr(hc_scale), _ptr(bias),
            T, n, D, sinkhorn_repeat, eps, n_splits, _stream(dev, stream))
    return _finish("mhc_pre_static", lib().mhc_pre_static, args, (post, comb, y), False, None)


def mhc_post(h, residual, post, comb, *, out=None, stream=None, prepare: bool = False):
    """out [T, n, D] = post_j * h + sum_i comb[i, j] * residual_i (prepare=True: a ``PreparedCall``)."""
    torch = _torch()
    T, n, D = residual.shape
    dev = _gpu_device(residual, "residual")
    dt = _dtype_code(residual)
    _check(h, (T, D), residual.dtype, dev, "h")
    _check(residual, (T, n, D), residual.dtype, dev, "residual")
    _check(post, (T, n), torch.float32, dev, "post")
    _check(comb, (T, n, n), torch.float32, dev, "comb")
    if out is None:
        with _on(stream):
            out = torch.empty_like(residual)
    _check(out, (T, n, D), residual.dtype, dev, "out")
    args = (_ptr(out), _ptr(h), _ptr(residual), _ptr(post), _ptr(comb), dt, T, n, D, _stream(dev, stream))
    return _finish("mhc_post", lib().mhc_post, args, out, prepare, (h, residual, post, comb))


def mhc_post_combine_norm(h, residual, post, comb, combine_w, norm_weight, *, norm_eps: float = 1e-6,
                          write_out: bool = True, normalized=None, out=None, stream=None, prepare: bool = False):
    """(normalized [T, D], out [T, n, D] or None): fused post mix + combine + RMSNorm (prepare=True: a
    ``PreparedCall``)."""
    torch = _torch()
    T, n, D = residual.shape
    dev = _gpu_device(residual, "residual")
    dt = _dtype_code(residual)
    _check(h, (T, D), residual.dtype, dev, "h")
    _check(residual, (T, n, D), residual.dtype, dev, "residual")
    _check(post, (T, n), torch.float32, dev, "post")
    _check(comb, (T, n, n), torch.float32, dev, "comb")
    _check(combine_w, (T, n), torch.float32, dev, "combine_w")
    _check(norm_weight, (D,), torch.float32, dev, "norm_weight")
    with _on(stream):
        normalized = torch.empty((T, D), dtype=residual.dtype, device=dev) if normalized is None else normalized
        if write_out:
            out = torch.empty_like(residual) if out is None else out
        else:
            out = None
    _check(normalized, (T, D), residual.dtype, dev, "normalized")
    if out is not None:
        _check(out, (T, n, D), residual.dtype, dev, "out")
    args = (_ptr(normalized), _ptr(out), _ptr(h), _ptr(residual), _ptr(post), _ptr(comb), _ptr(combine_w),
            _ptr(norm_weight), norm_eps, dt, T, n, D, _stream(dev, stream))
    return _finish("mhc_post_combine_norm", lib().mhc_post_combine_norm, args, (normalized, out), prepare,
                   (h, residual, post, comb, combine_w, norm_weight))


def mhc_post_pre_fused(T: int, n: int, D: int, n_splits: int = 0, dtype_code: int = MHC_BF16) -> bool:
    """True if mhc_post_pre runs as one launch for these sizes (with a 16-byte aligned fn)."""
    st = lib().mhc_post_pre_fused(T, n, D, n_splits, dtype_code)
    if st < 0:
        raise MhcError("mhc_post_pre_fused", st)
    return bool(st)


def mhc_post_pre(h, residual, post, comb, fn, hc_scale, bias, *, sinkhorn_repeat: int = 20, eps: float = 1e-6,
                 n_splits: int = 0, out=None, post_next=None, comb_next=None, y=None, workspace=None, stream=None,
                 prepare: bool = False):
    """(out [T, n, D], post' [T, n], comb' [T, n, n], y' [T, D]): mhc_post of the finished layer, then the
    next layer's mhc_pre (fn, hc_scale, bias) on its result (prepare=True: a ``PreparedCall``)."""
    torch = _torch()
    L = lib()
    T, n, D = residual.shape
    dev = _gpu_device(residual, "residual")
    dt = _dtype_code(residual)
    N = n * (n + 2)
    _check(h, (T, D), residual.dtype, dev, "h")
    _check(residual, (T, n, D), residual.dtype, dev, "residual")
    _check(post, (T, n), torch.float32, dev, "post")
    _check(comb, (T, n, n), torch.float32, dev, "comb")
    _check(fn, (n * D, N), torch.float32, dev, "fn")
    _check(hc_scale, (3,), torch.float32, dev, "hc_scale")
    _check(bias, (N,), torch.float32, dev, "bias")
    with _on(stream):
        out = torch.empty_like(residual) if out is None else out
        post_next = torch.empty((T, n), dtype=torch.float32, device=dev) if post_next is None else post_next
        comb_next = torch.empty((T, n, n), dtype=torch.float32, device=dev) if comb_next is None else comb_next
        y = torch.empty((T, D), dtype=residual.dtype, device=dev) if y is None else y
    if workspace is None:
        workspace = _default_workspace(L, T, n, D, n_splits, dt, dev, stream)
    _check(out, (T, n, D), residual.dtype, dev, "out")
    _check(post_next, (T, n), torch.float32, dev, "post_next")
    _check(comb_next, (T, n, n), torch.float32, dev, "comb_next")
    _check(y, (T, D), residual.dtype, dev, "y")
    args = (_ptr(out), _ptr(post_next), _ptr(comb_next), _ptr(y), _ptr(h), _ptr(residual), _ptr(post), _ptr(comb),
            dt, _ptr(fn), _ptr(hc_scale), _ptr(bias), T, n, D, sinkhorn_repeat, eps, n_splits, _ptr(workspace),
            _workspace_bytes(workspace, dev), _stream(dev, stream))
    return _finish("mhc_post_pre", L.mhc_post_pre, args, (out, post_next, comb_next, y), prepare,
                   (h, residual, post, comb, fn, hc_scale, bias, workspace))
