"""C ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments before any HIP call (so nothing launches)."""

import ctypes
import os
import re
import subprocess

import pytest

import mhc_hyper_connection_pre_amd as mhc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mhc.h")

OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE = 0, -1, -2, -3, -4
BF16, F32 = 0, 1
A = 0x100000          # a fake, 256-byte aligned "device" address: never dereferenced here


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"MHC_API\s+[\w\s\*]+?\b(mhc_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def L():
    # MHC_ABI_LIBRARY: another build of the same sources to run these checks on
    # (the host-sanitizer build of test_abi_hostsan.py)
    other = os.environ.get("MHC_ABI_LIBRARY")
    if other:
        return mhc.load_library(other)
    if not os.path.exists(mhc.library_path()):
        pytest.skip("libmhc.so not built")
    return mhc.lib()


def test_header_declares_the_boundary():
    syms = set(declared_symbols())
    assert {"mhc_pre", "mhc_post", "mhc_post_combine_norm", "mhc_post_pre", "mhc_pre_workspace_bytes",
            "mhc_pre_splits", "mhc_post_pre_fused", "mhc_status_string", "mhc_last_error"} <= syms


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", mhc.library_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, flags=re.M))
    for s in declared_symbols():
        assert s in exported, f"{s} declared in include/mhc.h but not exported"
        assert hasattr(L, s)
    # nothing but the C ABI is exported from the library's own code
    assert not [s for s in exported if s.startswith("_ZN3mhc")]


def test_status_strings(L):
    for st in (OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE, -5):
        assert L.mhc_status_string(st).decode().startswith("MHC_")
    assert L.mhc_status_string(42) == b"unknown mhc status"
    assert L.mhc_last_error() == b""


def pre(L, T=16, n=4, D=64, dt=BF16, post=A, comb=A + 0x10000, y=A + 0x20000, res=A + 0x30000, fn=A + 0x40000,
        hc=A + 0x50000, bias=A + 0x60000, repeat=20, eps=1e-6, splits=0, ws=A + 0x100000, ws_bytes=1 << 30):
    return L.mhc_pre(post, comb, y, res, dt, fn, hc, bias, T, n, D, repeat, eps, splits, ws, ws_bytes, None)


def test_pre_validation(L):
    assert pre(L, T=0) == OK                       # no-op, nothing launched
    assert pre(L, T=0, post=None, y=None) == OK
    assert pre(L, T=-1) == INVALID
    assert pre(L, n=0) == INVALID
    assert pre(L, n=5) == UNSUPPORTED
    assert pre(L, n=7) == UNSUPPORTED
    assert pre(L, n=9) == UNSUPPORTED
    assert pre(L, n=8, T=0) == OK                  # n = 8: built (two-pass path)
    assert pre(L, n=8, splits=-1) == UNSUPPORTED   # ... but not on the single-pass kernel
    assert pre(L, D=0) == INVALID
    assert pre(L, D=12) == MISALIGNED               # bf16 needs D % 8 == 0
    assert pre(L, D=12, dt=F32, T=0) == OK          # f32 needs D % 4 == 0
    assert pre(L, dt=7) == INVALID
    assert pre(L, repeat=0) == INVALID
    assert pre(L, eps=0.0) == INVALID
    assert pre(L, eps=float("nan")) == INVALID
    assert pre(L, splits=-257) == INVALID
    assert pre(L, splits=257) == INVALID
    assert pre(L, splits=-3) == UNSUPPORTED        # 3 slices do not divide D = 64 into 32-wide steps
    for k in ("post", "comb", "y", "res", "fn", "hc", "bias"):
        assert pre(L, **{k: None}) == INVALID, k
    assert pre(L, y=A + 8) == MISALIGNED
    assert pre(L, res=A + 2) == MISALIGNED
    assert pre(L, post=A + 2) == MISALIGNED
    assert pre(L, ws=None) == WORKSPACE
    assert pre(L, ws=A + 16) == WORKSPACE
    need = L.mhc_pre_workspace_bytes(16, 4, 64, 0, BF16)
    assert need > 0
    assert pre(L, ws_bytes=need - 1) == WORKSPACE
    # outputs that overlap another output, an input or the workspace
    assert pre(L, comb=A + 0x80) == INVALID                  # comb over post (256 B)
    assert pre(L, y=A + 0x30000 + 0x1000) == INVALID        # y inside the residual
    assert pre(L, post=A + 0x40000 + 0x5ff0) == INVALID     # post over the end of fn
    assert pre(L, y=A + 0x60000 - 0x7f0) == INVALID         # y runs into bias
    assert pre(L, post=A + 0x100000 + 0x200) == INVALID     # post inside the workspace
    assert pre(L, ws=A + 0x10000 + 0x300, ws_bytes=need) == INVALID   # workspace over the end of comb


HUGE = [(2**62, 4, 64), (16, 4, 2**60), (2**40, 4, 2**40), (2**63 - 1, 1, 8), (16, 4, 2**63 - 8),
        (2**31, 4, 7168), (1, 2**31 - 1, 8)]


@pytest.mark.parametrize("T,n,D", HUGE, ids=str)
def test_sizes_near_the_integer_limits_are_refused(L, T, n, D):
    """Element counts that overflow 64 bits, or pass the 32-bit lane offsets the kernels use, are refused
    before any arithmetic on them can overflow (the host-sanitizer build runs these too)."""
    assert pre(L, T=T, n=n, D=D) == UNSUPPORTED
    assert L.mhc_pre_workspace_bytes(T, n, D, 0, BF16) == 0
    assert L.mhc_pre_splits(T, n, D, 0, BF16) == UNSUPPORTED
    assert L.mhc_post_pre_fused(T, n, D, 0, BF16) == UNSUPPORTED
    assert L.mhc_post(A, A + 0x10000, A + 0x20000, A + 0x30000, A + 0x40000, BF16, T, n, D, None) < 0
    assert L.mhc_post_combine_norm(A, None, A + 0x10000, A + 0x20000, A + 0x30000, A + 0x40000, A + 0x50000,
                                   A + 0x60000, 1e-6, BF16, T, n, D, None) < 0
    assert L.mhc_pre_splits(16, 4, 64, -2**31, BF16) == INVALID
    assert L.mhc_pre_splits(16, 4, 64, 2**31 - 1, BF16) == INVALID


def test_pre_static_validation(L):
    """The no-allocation variant: its size limit and mhc_pre's own argument checks, before any launch."""
    L.mhc_pre_static.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] + [ctypes.c_void_p] * 3 + [
        ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    L.mhc_pre_static.restype = ctypes.c_int

    def st(T=16, n=4, D=64, dt=BF16, splits=0, post=A, repeat=20):
        return L.mhc_pre_static(post, A + 0x10000, A + 0x20000, A + 0x30000, dt, A + 0x40000, A + 0x50000,
                                A + 0x60000, T, n, D, repeat, 1e-6, splits, None)

    limit = 32 << 20
    assert L.mhc_pre_workspace_bytes(2048, 4, 7168, 0, BF16) <= limit     # the throughput shape fits
    assert L.mhc_pre_workspace_bytes(16384, 4, 7168, 0, BF16) > limit     # the 16384-token prefill does not
    assert st(T=16384, D=7168) == WORKSPACE
    assert b"32 MiB" in L.mhc_last_error()
    assert st(T=0) == OK
    assert st(n=5) == UNSUPPORTED
    assert st(D=12) == MISALIGNED
    assert st(repeat=0) == INVALID
    assert st(T=-1) == INVALID


def test_pre_plan(L):
    # split count: explicit values honoured (capped at the number of 32-wide k-steps), auto is positive
    assert L.mhc_pre_splits(2048, 4, 4096, 1, BF16) == 1
    assert L.mhc_pre_splits(16384, 4, 7168, 4, BF16) == 4
    assert L.mhc_pre_splits(16384, 4, 7168, 8, BF16) == 8
    assert L.mhc_pre_splits(2048, 4, 7168, 0, BF16) >= 1
    assert L.mhc_pre_splits(1, 1, 8, 64, BF16) == 1              # K = 8: one k-step
    assert L.mhc_pre_splits(1, 5, 8, 0, BF16) == UNSUPPORTED
    assert L.mhc_pre_workspace_bytes(0, 4, 64, 0, BF16) == 0
    assert L.mhc_pre_workspace_bytes(16, 5, 64, 0, BF16) == 0
    # two-pass workspace: 256 B of status words, packed fn (K/32 k-steps x 4
    # column blocks x 1 KiB), partials [S, T, 28] fp32
    T, n, D = 2048, 4, 7168
    fnp = (n * D // 32) * 4 * 1024      # [hi | lo | lo2 of the 4 pre columns] = 52 -> 4 blocks of 16
    ws16 = L.mhc_pre_workspace_bytes(T, n, D, 16, BF16)
    assert L.mhc_pre_splits(T, n, D, 16, BF16) == 16
    assert ws16 == 256 + (fnp + 255) // 256 * 256 + (16 * T * 28 * 4 + 255) // 256 * 256
    # single-pass workspace (n_splits = -1, and the library's choice for bf16
    # when D % 32 == 0): status, packed fn, then 8-byte tagged words: partials
    # [S, T, 25] and pre [T, 4]
    S = L.mhc_pre_splits(T, n, D, -1, BF16)
    assert S > 0 and D % S == 0 and (D // S) % 32 == 0
    assert L.mhc_pre_splits(T, n, D, 0, BF16) == S
    wsS = L.mhc_pre_workspace_bytes(T, n, D, -1, BF16)
    assert wsS == 256 + fnp + (S * T * 25 * 8 + 255) // 256 * 256 + T * 4 * 8
    assert L.mhc_pre_splits(T, n, 104, -1, BF16) == UNSUPPORTED        # D % 32 != 0
    assert L.mhc_pre_splits(T, n, 104, 0, BF16) >= 1                    # ... two-pass instead
    assert L.mhc_pre_splits(8, 4, 256, -1, F32) == UNSUPPORTED           # fp32: two-pass only
    assert L.mhc_pre_splits(T, n, D, -257, BF16) == INVALID
    # explicit single-pass slice counts: D = 32 * cps * S for a built cps, else unsupported
    for S_ in (32, 56, 112):
        assert L.mhc_pre_splits(T, n, D, -S_, BF16) == S_
        assert L.mhc_pre_workspace_bytes(T, n, D, -S_, BF16) == 256 + fnp + (S_ * T * 25 * 8 + 255) // 256 * 256 + T * 4 * 8
    assert L.mhc_pre_splits(T, n, D, -16, BF16) == UNSUPPORTED       # cps 14: its residual slice needs too many registers
    assert L.mhc_pre_splits(T, n, D, -28, BF16) == UNSUPPORTED       # cps 8: its fn fragments do not fit in LDS
    assert L.mhc_pre_splits(T, n, D, -2, BF16) == UNSUPPORTED        # cps 112 is not built
    # slices of three and six columns: D = 3072 and 6144 take 32 slices (two generations at T = 2048)
    assert L.mhc_pre_splits(T, 4, 6144, -1, BF16) == 32
    assert L.mhc_pre_splits(T, 3, 3072, -32, BF16) == 32
    assert L.mhc_pre_splits(T, 4, 6144, -48, BF16) == 48               # cps 4 still accepted
    assert L.mhc_post_pre_fused(T, 4, 6144, -32, BF16) == 1           # 4 n cps + 4 cps = 120 registers
    assert L.mhc_pre_splits(T, n, 104, -1, F32) == UNSUPPORTED
    # fp32 residuals always take the two-pass path (no packed fn)
    assert L.mhc_pre_workspace_bytes(8, 4, 256, 0, F32) == 256 + (L.mhc_pre_splits(8, 4, 256, 0, F32) * 8 * 28 * 4 + 255) // 256 * 256
    # n = 8 (N = 80): two-pass only; [hi | lo | lo2 of the 8 pre columns] = 168 -> 11 blocks; partials [S, T, 84]
    T8, D8 = 64, 1024
    assert L.mhc_pre_splits(T8, 8, D8, -1, BF16) == UNSUPPORTED
    S8 = L.mhc_pre_splits(T8, 8, D8, 0, BF16)
    assert S8 >= 1 and L.mhc_pre_splits(T8, 8, D8, 4, BF16) == 4
    fnp8 = (8 * D8 // 32) * 11 * 1024
    assert L.mhc_pre_workspace_bytes(T8, 8, D8, 4, BF16) == 256 + fnp8 + (4 * T8 * 84 * 4 + 255) // 256 * 256
    assert L.mhc_post_pre_fused(T8, 8, D8, 0, BF16) == 0


def test_post_validation(L):
    def post(T=4, n=4, D=64, dt=BF16, out=A, h=A + 0x10000, res=A + 0x20000, p=A + 0x30000, c=A + 0x40000):
        return L.mhc_post(out, h, res, p, c, dt, T, n, D, None)
    assert post(T=0) == OK
    assert post(T=-3) == INVALID
    assert post(n=5) == UNSUPPORTED
    assert post(n=8, T=0) == OK
    assert post(D=4) == MISALIGNED
    assert post(out=None) == INVALID
    assert post(h=A + 4) == MISALIGNED
    assert post(c=A + 1) == MISALIGNED
    assert post(res=A + 0x7f0) == INVALID      # out (2 KB) runs into the residual
    assert post(h=A) == INVALID                # out over h
    assert post(out=A + 0x30000 - 0x10) == INVALID   # out over post


def test_post_pre_validation(L):
    B = 0x100000
    def pp(T=4, n=4, D=64, dt=BF16, out=B, pn=B + 0x10000, cn=B + 0x20000, y=B + 0x30000, h=B + 0x40000,
           res=B + 0x50000, p=B + 0x60000, c=B + 0x70000, fn=B + 0x80000, hc=B + 0x90000, bias=B + 0xA0000,
           R=20, eps=1e-6, sp=0, ws=None, wsb=0):
        return L.mhc_post_pre(out, pn, cn, y, h, res, p, c, dt, fn, hc, bias, T, n, D, R, eps, sp, ws, wsb, None)
    assert pp(T=0) == OK
    assert pp(T=-1) == INVALID
    assert pp(n=5) == UNSUPPORTED
    assert pp(D=12) == MISALIGNED
    assert pp(R=0) == INVALID
    assert pp(eps=0.0) == INVALID
    assert pp(sp=-257) == INVALID
    assert pp(sp=-3) == UNSUPPORTED              # no single-pass tiling with 3 slices of D = 64
    assert pp(dt=F32, sp=-1) == UNSUPPORTED      # the single-pass kernel is bf16 only
    assert pp(h=None) == INVALID
    assert pp(fn=None) == INVALID
    need = L.mhc_pre_workspace_bytes(4, 4, 64, 0, BF16)
    W = B + 0x200000
    assert pp(out=B + 0x50000, ws=W, wsb=need) == INVALID        # out over the residual
    assert pp(out=B + 0x40000 - 64, ws=W, wsb=need) == INVALID   # out over h
    assert pp(y=B + 0x40000, ws=W, wsb=need) == INVALID          # y_next over h
    assert pp(cn=B + 0x10000 + 16, ws=W, wsb=need) == INVALID    # comb_next over post_next
    assert pp(pn=W + 0x100, ws=W, wsb=need) == INVALID           # post_next inside the workspace
    assert pp(y=B + 0x90000, ws=W, wsb=need) == INVALID          # y_next over hc_scale
    assert pp(y=B + 0x30008) == MISALIGNED
    assert pp(c=B + 0x70001) == MISALIGNED
    assert pp() == WORKSPACE                     # no workspace
    need = L.mhc_pre_workspace_bytes(4, 4, 64, 0, BF16)
    assert need > 0
    assert pp(ws=B + 0x200000 + 8, wsb=need) == WORKSPACE   # not 256-byte aligned
    assert pp(ws=B + 0x200000, wsb=need - 1) == WORKSPACE
    assert L.mhc_post_pre_fused(2048, 4, 7168, 0, BF16) in (0, 1)
    assert L.mhc_post_pre_fused(8, 4, 256, 0, F32) == 0
    assert L.mhc_post_pre_fused(8, 4, 256, 3, BF16) == 0
    assert L.mhc_post_pre_fused(8, 5, 256, 0, BF16) == UNSUPPORTED


def test_post_combine_norm_validation(L):
    def pcn(T=4, n=4, D=64, dt=BF16, nz=A, out=A + 0x10000, h=A + 0x20000, res=A + 0x30000, p=A + 0x40000,
            c=A + 0x50000, w=A + 0x60000, g=A + 0x70000, eps=1e-6):
        return L.mhc_post_combine_norm(nz, out, h, res, p, c, w, g, eps, dt, T, n, D, None)
    assert pcn(T=0) == OK
    assert pcn(T=0, out=None) == OK
    assert pcn(n=6) == UNSUPPORTED
    assert pcn(n=8, T=0) == OK
    assert pcn(eps=0.0) == INVALID
    assert pcn(nz=None) == INVALID
    assert pcn(w=None) == INVALID
    assert pcn(out=A + 8) == MISALIGNED
    assert pcn(nz=A + 0x20000) == INVALID      # normalized over h
    assert pcn(out=A + 0x100) == INVALID       # out_residual over normalized
    assert pcn(nz=A + 0x70000 + 0x80) == INVALID   # normalized over norm_weight
    assert pcn(D=8 * 4097) == UNSUPPORTED          # more than 1024 threads x 4 vectors
    assert pcn(D=8 * 4096, T=0) == OK
    assert pcn(n=8, D=8 * 2049) == UNSUPPORTED     # n = 8: 512 threads x 4 vectors
    assert pcn(n=8, D=8 * 2048, T=0) == OK
    assert pcn(n=8, D=4 * 2049, dt=F32) == UNSUPPORTED


def test_binding_raises_without_gpu_tensors(L):
    import torch
    x = torch.zeros((2, 4, 8), dtype=torch.bfloat16)
    # tensors that live in host memory are refused before any call
    with pytest.raises(ValueError, match="GPU"):
        mhc.mhc_post(x[:, 0].float(), x, torch.zeros(2, 4), torch.zeros(2, 4, 4))
    h, p, c = x[:, 0].contiguous(), torch.zeros(2, 4), torch.zeros(2, 4, 4)
    fn, hc, b = torch.zeros(32, 24), torch.ones(3), torch.zeros(24)
    with pytest.raises(ValueError, match="GPU"):
        mhc.mhc_post(h, x, p, c)
    with pytest.raises(ValueError, match="GPU"):
        mhc.mhc_pre(x, fn, hc, b)
    with pytest.raises(ValueError, match="GPU"):
        mhc.mhc_pre(x, fn, hc, b, prepare=True)
    with pytest.raises(ValueError, match="GPU"):
        mhc.mhc_post_pre(h, x, p, c, fn, hc, b)
    with pytest.raises(ValueError, match="GPU"):
        mhc.mhc_post_combine_norm(h, x, p, c, torch.zeros(2, 4), torch.ones(8))
    with pytest.raises(ValueError, match="GPU"):
        mhc.mhc_pre_sync_timeouts(torch.zeros(256, dtype=torch.uint8), x)


def test_pre_plan_info(L, monkeypatch):
    import json
    info = (ctypes.c_int * 5)()
    assert L.mhc_pre_plan_info(2048, 4, 7168, 0, BF16, 0, None) == INVALID
    assert L.mhc_pre_plan_info(1, 5, 8, 0, BF16, 0, info) == UNSUPPORTED
    assert L.mhc_pre_plan_info(2048, 4, 7168, -257, BF16, 0, info) == INVALID
    monkeypatch.delenv("MHC_STAGGER", raising=False)
    # every measured point of the tile table: the plan takes the entry's tiling and instance
    table = json.load(open(os.path.join(ROOT, "mhc_hyper_connection_pre_amd", "tile_table.json")))
    for e in table["entries"]:
        for p in e["points"]:
            args = (p["T"], e["n"], e["D"], 0, e["dt"], 1 if e["op"] == "boundary" else 0)
            assert L.mhc_pre_plan_info(*args, info) == OK, args
            got = list(info)
            if p["best"] < 0:
                S = -p["best"]
                assert got[:2] == [1, S] and got[2] * 32 * S == e["D"], (args, got)
                assert got[3] >= 1, (args, got)
                assert got[4] == p["stagger"], (args, got, p)
            else:
                assert got == [0, p["best"], 0, 0, -1], (args, got)
            if e["op"] == "pre":
                assert L.mhc_pre_splits(*args[:5]) == abs(p["best"]), args
    # explicit knobs: a single-pass slice count and a two-pass split count
    assert L.mhc_pre_plan_info(2048, 4, 7168, -56, BF16, 0, info) == OK and list(info)[:3] == [1, 56, 4]
    assert L.mhc_pre_plan_info(2048, 4, 7168, 8, BF16, 0, info) == OK and list(info) == [0, 8, 0, 0, -1]
    assert L.mhc_pre_plan_info(64, 4, 256, 0, F32, 0, info) == OK and info[0] == 0 and info[4] == -1
    # the instance follows MHC_STAGGER when it is set, for either step
    for boundary in (0, 1):
        for v in ("0", "1"):
            monkeypatch.setenv("MHC_STAGGER", v)
            assert L.mhc_pre_plan_info(2048, 4, 7168, -32, BF16, boundary, info) == OK
            assert list(info)[:3] == [1, 32, 7] and info[4] == int(v)
    # without the table (an explicit slice count): the rule, by generations of resident tiles
    monkeypatch.delenv("MHC_STAGGER")
    assert L.mhc_pre_plan_info(128, 4, 7168, -32, BF16, 0, info) == OK and info[3] == 1 and info[4] == 0
    assert L.mhc_pre_plan_info(16384, 4, 7168, -32, BF16, 1, info) == OK and info[3] >= 12 and info[4] == 1
