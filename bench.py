#!/usr/bin/env python3
"""Benchmark of the mHC layer-boundary hot path on one MI355X.

One step = mhc_pre on a [T, n, D] residual followed by mhc_post on the same
residual with the block output h, using the post/comb that pre produced. The
default workload is prefill with T = 2048 tokens, n = 4 streams, D = 7168
(bf16), fn fp32 [28672, 24]. Inputs are seeded synthetic data already
resident in HBM when the timed region starts. Steps rotate over input and
output buffer sets such that the other sets move at least twice the 256 MB
Infinity Cache between two uses of one (three sets at the prefill sizes), so
no step reads inputs an earlier step left there; decode-sized sets stay
cached whatever the rotation.

Timing (the headline): K steps, each pre and each post call timed alone by
HIP events on its launch stream (without the system-scope fence) after a
read of 1 GiB that evicts the L2s and the 256 MB Infinity Cache, so every
call reads its inputs from HBM, as in a model, where the block between a
layer's pre and post evicts the residual; ms_per_step is the mean pre call
plus the mean post call, value = T / ms_per_step. Each buffer set's calls
are prepared once by the binding, so a call's host work is the C call
itself. Then, as extra fields: the same steps back to back with nothing
between the launches ("back_to_back": post then finds part of the residual
in the memory-side cache), and the layer boundary as one call, mhc_post_pre
(post of one layer, then the next layer's pre), back to back and after the
sweep ("boundary"); at decode sizes also sixteen boundary calls captured in
one HIP graph ("graph_of_16_us_per_call").

Prints one JSON line: tokens/s (value), algorithmic HBM GB/s and its fraction
of the 8 TB/s peak, a roofline object for the dominant kernel (algorithmic
bytes per launch / mean launch duration from the events; the pre call, with
the post call beside it as roofline_tail), the boundary call, the SHA-256 of
every input array, the host's CPU model, the source revision, and the CPU
oracle timed on the host as a baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       python bench.py --summarize-rocprof DIR   (summarise rocprofv3 output)
       python bench.py --write-traffic FETCH_DIR WRITE_DIR   (traffic profiles from two counter passes)
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "mhc_pre+post tokens/s and HBM GB/s (% of peak), T=2048 n=4 D=7168"
PEAK_HBM_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "mhc_hyper_connection_pre_amd", "csrc")
# Counter-derived HBM traffic per launch of the two kernels of the default
# workload: the profile file and the sources its number holds for.
_RESIDENT_SOURCES = ["mhc_pre_resident.hip", "mhc_device.h", "mhc_pack.h", "mhc_epilogue.h", "mhc_internal.h"]
TRAFFIC = {
    "pre": ("traffic_pre_resident_prefill-d7168.txt", "pre_resident_kernel<4, 7, false,", _RESIDENT_SOURCES),
    "post": ("traffic_post_prefill-d7168.txt", "post_kernel<", ["mhc_post.hip", "mhc_device.h"]),
    "boundary": ("traffic_boundary_prefill-d7168.txt", "pre_resident_kernel<4, 7, true,", _RESIDENT_SOURCES),
}
COPY_KIB = 1 << 20   # the 1 GiB calibration copy bench.py runs, in KiB read and written


# ---------------------------------------------------------------- algorithmic bytes

def pre_bytes(T, n, D, e):
    """Every input read once, every output written once: residual, fn, hc_scale + bias, y, post + comb."""
    N = n * (n + 2)
    return T * n * D * e + n * D * N * 4 + (N + 3) * 4 + T * D * e + T * (n + n * n) * 4


def post_bytes(T, n, D, e):
    """h, residual, post + comb read once; out written once."""
    return T * D * e + T * n * D * e + T * (n + n * n) * 4 + T * n * D * e


def boundary_bytes(T, n, D, e):
    """mhc_post_pre: h, residual, post, comb, the next layer's fn, hc_scale and bias read once; out, y, post
    and comb of the next layer written once (out is never read back)."""
    N = n * (n + 2)
    return (T * D * e + T * n * D * e + T * (n + n * n) * 4 + n * D * N * 4 + (N + 3) * 4
            + T * n * D * e + T * D * e + T * (n + n * n) * 4)


def pcn_bytes(T, n, D, e):
    """Fused post + combine + RMSNorm writing both outputs: h, residual, post, comb, combine_w and the norm
    weight read once; normalized [T, D] and out [T, n, D] written once."""
    return T * D * e + T * n * D * e + T * (n + n * n) * 4 + T * n * 4 + D * 4 + T * D * e + T * n * D * e


# ---------------------------------------------------------------- traffic from counters

def code_text(src: str) -> str:
    """C++ source without comments and with whitespace runs collapsed: edits to comments keep the hash."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_hash(which, read=None):
    """Hash of the code (comments excluded) of the sources a traffic profile depends on."""
    h = hashlib.sha256()
    for name in TRAFFIC[which][2]:
        if read is None:
            with open(os.path.join(CSRC, name)) as f:
                text = f.read()
        else:
            text = read(name)
        h.update(code_text(text).encode())
    return h.hexdigest()[:16]


def stored_traffic(which):
    """Counter-derived HBM bytes per launch, if measured on the current kernel sources."""
    path = os.path.join(PROFILES, TRAFFIC[which][0])
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != source_hash(which):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def counter_values(d, counter):
    """{kernel name: [value per dispatch]} for one counter from a rocprofv3 --pmc output directory."""
    out = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


# the counter passes behind the traffic profiles (recorded in each profile unless --traffic-command is given)
TRAFFIC_COMMAND = [
    "export TMPDIR=/tmp; R=$PWD; cd /tmp",
    "timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE -d $R/gpurun_out/pmc_fetch -o f --output-format csv -- "
    "python3 $R/bench.py --steps 4 --warmup 2 --no-cpu-baseline",
    "timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE -d $R/gpurun_out/pmc_write -o w --output-format csv -- "
    "python3 $R/bench.py --steps 4 --warmup 2 --no-cpu-baseline",
    "cd $R; python3 bench.py --write-traffic gpurun_out/pmc_fetch gpurun_out/pmc_write",
]


def write_traffic(fetch_dir, write_dir, command):
    """Write the traffic profiles of the pre and post kernels from a FETCH_SIZE and a WRITE_SIZE pass over
    the default bench run. Each counter is scaled by what it reads for the 1 GiB copy the same run makes
    (the largest __amd_rocclr_copyBuffer dispatch)."""
    fetch, write = counter_values(fetch_dir, "FETCH_SIZE"), counter_values(write_dir, "WRITE_SIZE")
    copy = [k for k in fetch if "copyBuffer" in k]
    if not copy:
        raise SystemExit("no copy kernel in the FETCH_SIZE pass: cannot calibrate")
    fs = COPY_KIB / max(fetch[copy[0]])
    ws = COPY_KIB / max(write[copy[0]])
    T, n, D, e = 2048, 4, 7168, 2
    algo = {"pre": pre_bytes(T, n, D, e), "post": post_bytes(T, n, D, e), "boundary": boundary_bytes(T, n, D, e)}
    for which, (fname, key, sources) in TRAFFIC.items():
        names = [k for k in fetch if key in k]
        if not names or names[0] not in write:
            raise SystemExit(f"kernel {key} missing from the counter passes")
        k = names[0]
        f_kib, w_kib = sum(fetch[k]) / len(fetch[k]), sum(write[k]) / len(write[k])
        total = f_kib * 1024 * fs + w_kib * 1024 * ws
        with open(os.path.join(PROFILES, fname), "w") as f:
            f.write(f"# HBM traffic of {k}, prefill T=2048 n=4 D=7168 bf16, per launch\n")
            f.write("# two rocprofv3 counter passes (one counter each), from the repository root on an MI355X:\n")
            for line in command or TRAFFIC_COMMAND:
                f.write(f"#   {line}\n")
            f.write(f"# calibration: the 1 GiB copy reads FETCH_SIZE {max(fetch[copy[0]]):.0f} KiB and WRITE_SIZE "
                    f"{max(write[copy[0]]):.0f} KiB per dispatch: scales {fs:.5f} and {ws:.5f}\n")
            f.write(f"# {len(fetch[k])} dispatches: FETCH_SIZE {f_kib:.1f} KiB = {f_kib * 1024 * fs / 1e6:.1f} MB read, "
                    f"WRITE_SIZE {w_kib:.1f} KiB = {w_kib * 1024 * ws / 1e6:.1f} MB written\n")
            f.write(f"# algorithmic bytes per launch: {algo[which]} ({algo[which] / 1e6:.1f} MB)\n")
            f.write(f"# sources: {', '.join(sources)} (the hash covers their code, comments excluded)\n")
            f.write(f"kernel_source_sha256_16: {source_hash(which)}\n")
            f.write(f"fetch_scale: {fs:.5f}\nwrite_scale: {ws:.5f}\n")
            f.write(f"hbm_bytes_per_launch: {total:.0f}\n")
        print(f"{fname}: {total / 1e6:.1f} MB per launch (algorithmic {algo[which] / 1e6:.1f} MB)")


def summarize_rocprof(d, warmup=None, steps=None):
    """Print per-kernel averages from a rocprofv3 output directory (kernel trace and/or counters).

    With warmup W and steps K (the bench run's own): for each kernel also the average over its dispatches
    W .. W + K - 1 in start order, the headline pass of bench.py, where each pre and post call runs after a
    cache sweep ("headline_avg_us")."""
    rows = {}
    for path in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            rows.setdefault(r["Name"], {}).update(
                {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                 "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
                 "total_us": float(r["TotalDurationNs"]) / 1e3, "pct": float(r["Percentage"])})
    if warmup is not None and steps is not None:
        disp = {}
        for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                disp.setdefault(r["Kernel_Name"], []).append(
                    (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        for k, v in disp.items():
            v.sort()
            sel = [dur for _, dur in v[warmup:warmup + steps]]
            if len(sel) == steps:
                rows.setdefault(k, {})["headline_avg_us"] = sum(sel) / len(sel) / 1e3
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        acc = {}
        for r in csv.DictReader(open(path)):
            key = (r["Kernel_Name"], r["Counter_Name"])
            acc.setdefault(key, []).append(float(r["Counter_Value"]))
        for (k, c), v in acc.items():
            rows.setdefault(k, {})[c + "_avg"] = sum(v) / len(v)
            rows.setdefault(k, {})[c + "_n"] = len(v)
    for k, v in sorted(rows.items(), key=lambda kv: -kv[1].get("total_us", 0)):
        print(json.dumps({"kernel": k, **v}))


# ---------------------------------------------------------------- provenance

def host_info():
    """CPU model and the CPUs this process may use."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "cpus_available": len(os.sched_getaffinity(0))}


def revision_info():
    """The git revision when the tree has its history, and a hash of the product sources either way (a GPU
    box runs a copy of the tree without .git)."""
    import subprocess
    rev = None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        rev = r.stdout.strip() or None if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        rev = None
    h = hashlib.sha256()
    for d in (CSRC, os.path.join(ROOT, "include")):
        for name in sorted(os.listdir(d)):
            if name.endswith((".hip", ".cpp", ".h")):
                with open(os.path.join(d, name), "rb") as f:
                    h.update(name.encode() + b"\0" + f.read())
    with open(os.path.abspath(__file__), "rb") as f:
        h.update(b"bench.py\0" + f.read())
    out = {"git": rev, "sources_sha256_16": h.hexdigest()[:16]}
    # the revision the library was built from, recorded by the build beside it
    path = os.path.join(ROOT, "mhc_hyper_connection_pre_amd", "libmhc.revision")
    if os.path.exists(path):
        vals = dict(line.split(": ", 1) for line in open(path).read().splitlines() if ": " in line)
        out["library_built_from_git"] = None if vals.get("git") in (None, "None") else vals["git"]
        out["library_tree_had_uncommitted_changes"] = {"True": True, "False": False}.get(vals.get("dirty"))
    return out


# ---------------------------------------------------------------- timing events

class HipEvents:
    """HIP events without the system-scope fence, recorded on a given stream (per-kernel durations)."""

    def __init__(self, stream_handle, count):
        import ctypes
        self._c = ctypes
        self._hip = ctypes.CDLL("libamdhip64.so")   # the HIP runtime torch has loaded
        self._hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._stream = ctypes.c_void_p(stream_handle)
        self._ev = []
        for _ in range(count):
            e = ctypes.c_void_p()
            if self._hip.hipEventCreateWithFlags(ctypes.byref(e), 0x20000000) != 0:   # hipEventDisableSystemFence
                raise RuntimeError("hipEventCreateWithFlags failed")
            self._ev.append(e)

    def record(self, i):
        if self._hip.hipEventRecord(self._ev[i], self._stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i, j):
        f = self._c.c_float()
        if self._hip.hipEventElapsedTime(self._c.byref(f), self._ev[i], self._ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def destroy(self):
        for e in self._ev:
            self._hip.hipEventDestroy(e)
        self._ev = []


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(x, min_seconds):
    """The float64 oracle (as it stands) on the same workload, repeated until min_seconds elapse."""
    import numpy as np
    import oracle.mhc_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report one thread per BLAS call
        blas = 1
    s = x.spec
    reps, t_total = 0, 0.0
    while t_total < min_seconds or reps == 0:
        t0 = time.perf_counter()
        post, comb, y = O.mhc_pre(x.residual, x.fn, x.hc_scale, x.bias, n=s.n, D=s.D, dtype=s.dtype,
                                  sinkhorn_repeat=s.sinkhorn_repeat, eps=s.eps)
        if s.combine and s.dtype == "bf16":
            O.mhc_post_combine_norm(x.h, x.residual, post, comb, x.combine_w, x.norm_weight, n=s.n, D=s.D,
                                    dtype=s.dtype, norm_eps=s.norm_eps)
        else:
            O.mhc_post(x.h, x.residual, post, comb, n=s.n, D=s.D, dtype=s.dtype)
        t_total += time.perf_counter() - t0
        reps += 1
        if reps >= 20:
            break
    del np
    return {"value": reps * s.T / t_total, "unit": "tokens/s", "cores": int(blas), "kind": "oracle",
            "sample": f"full workload ({s.T} tokens) x {reps} repetition(s), {t_total:.1f} s; float64 numpy, "
                      f"matmul on {blas} BLAS thread(s), elementwise single-threaded",
            "host_cpus_available": len(os.sched_getaffinity(0))}


# ---------------------------------------------------------------- GPU benchmark

def run(args):
    import numpy as np
    import torch

    import mhc_hyper_connection_pre_amd as mhc
    from mhc_hyper_connection_pre_amd import workloads as W

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (torch.cuda.is_available() is False)")
    dev = torch.device("cuda:0")
    spec = W.spec(args.workload)
    if args.n_splits is not None:
        spec = W.spec(args.workload, n_splits=args.n_splits)
    x = W.generate(spec)
    T, n, D = spec.T, spec.n, spec.D
    tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    e = 2 if spec.dtype == "bf16" else 4

    def dev_t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    fn, hc, bias = dev_t(x.fn), dev_t(x.hc_scale), dev_t(x.bias)
    # decode workloads end the step with the fused post + combine + RMSNorm
    fused_tail = spec.combine and spec.dtype == "bf16"
    if fused_tail:
        cw, nw = dev_t(x.combine_w), dev_t(x.norm_weight)
    tail_bytes = pcn_bytes if fused_tail else post_bytes
    per_set = pre_bytes(T, n, D, e) + tail_bytes(T, n, D, e)
    # Between two uses of a buffer set the other sets move at least twice the
    # 256 MB Infinity Cache (with two sets of this workload's 292 MB, pre read
    # residual lines the step before last had left there: 45.5 against
    # 49.3 us). Decode-sized sets stay cached whatever the rotation.
    nsets = max(3, min(8, -(-int(2 * 256e6) // max(per_set, 1)) + 1))
    if args.sets:
        nsets = args.sets
    sets = []
    for k in range(nsets):
        res = dev_t(x.residual) if k == 0 else sets[0]["residual"].clone()
        h = dev_t(x.h) if k == 0 else sets[0]["h"].clone()
        sets.append({
            "residual": res, "h": h,
            "post": torch.empty((T, n), dtype=torch.float32, device=dev),
            "comb": torch.empty((T, n, n), dtype=torch.float32, device=dev),
            "y": torch.empty((T, D), dtype=tdt, device=dev),
            "out": torch.empty((T, n, D), dtype=tdt, device=dev),
            "normalized": torch.empty((T, D), dtype=tdt, device=dev),
        })
    ws_bytes = mhc.mhc_pre_workspace_bytes(T, n, D, spec.n_splits, 0 if spec.dtype == "bf16" else 1)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    ws[:256].zero_()   # status words of a fresh workspace
    S = mhc.mhc_pre_splits(T, n, D, spec.n_splits, 0 if spec.dtype == "bf16" else 1)
    try:
        single = spec.n_splits <= 0 and mhc.mhc_pre_splits(T, n, D, -1, 0 if spec.dtype == "bf16" else 1) == S
    except mhc.MhcError:
        single = False
    stream = torch.cuda.current_stream(dev)

    def call_pre(b, st, prepare=False):
        return mhc.mhc_pre(b["residual"], fn, hc, bias, sinkhorn_repeat=spec.sinkhorn_repeat, eps=spec.eps,
                           n_splits=spec.n_splits, post=b["post"], comb=b["comb"], y=b["y"], workspace=ws, stream=st,
                           prepare=prepare)

    def call_post(b, st, prepare=False):
        if fused_tail:
            return mhc.mhc_post_combine_norm(b["h"], b["residual"], b["post"], b["comb"], cw, nw,
                                             norm_eps=spec.norm_eps, normalized=b["normalized"], out=b["out"],
                                             stream=st, prepare=prepare)
        return mhc.mhc_post(b["h"], b["residual"], b["post"], b["comb"], out=b["out"], stream=st, prepare=prepare)

    for i in range(args.warmup):
        call_pre(sets[i % nsets], stream)
        call_post(sets[i % nsets], stream)
    torch.cuda.synchronize()

    if not args.graph:
        # each buffer set's calls checked and marshalled once by the binding
        # (PreparedCall): a step then costs the host about what the C calls
        # take, not the binding's per-call checks (several us, more than a
        # decode-sized kernel)
        prep_pre = [call_pre(sets[k], stream, True) for k in range(nsets)]
        prep_post = [call_post(sets[k], stream, True) for k in range(nsets)]

        def run_pre(k):
            prep_pre[k]()

        def run_post(k):
            prep_post[k]()
    else:
        # Every call of a step captured once per buffer set: a replay launches the
        # same kernels with no host work per kernel (the single-pass path keeps
        # its per-call state in the workspace, so replays are independent calls).
        graphs = []
        for k in range(nsets):
            gp, gq = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(gp):
                call_pre(sets[k], torch.cuda.current_stream(dev))
            with torch.cuda.graph(gq):
                call_post(sets[k], torch.cuda.current_stream(dev))
            graphs.append((gp, gq))
        for k in range(nsets):   # warm replays
            graphs[k][0].replay()
            graphs[k][1].replay()
        torch.cuda.synchronize()

        def run_pre(k):
            graphs[k][0].replay()

        def run_post(k):
            graphs[k][1].replay()

    # The headline: K steps, each call timed alone after a read of 1 GiB
    # (four times the 256 MB Infinity Cache, far more than the L2s hold), so
    # every call reads its inputs from HBM, as in a model, where the block
    # between a layer's pre and post evicts the residual. HIP events without
    # the system-scope fence bracket each call on its launch stream (a default
    # event writes back and invalidates the caches, which slows the kernel
    # after it); the sweep sits outside them. It only reads: a sweep that
    # writes leaves dirty lines whose write-back then lands in the timed call.
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    ev = HipEvents(stream.cuda_stream, 4 * args.steps)
    torch.cuda.synchronize()
    th0 = time.perf_counter()
    for i in range(args.steps):
        flush.max()
        ev.record(4 * i)
        run_pre(i % nsets)
        ev.record(4 * i + 1)
        flush.max()
        ev.record(4 * i + 2)
        run_post(i % nsets)
        ev.record(4 * i + 3)
    torch.cuda.synchronize()
    headline_wall_s = time.perf_counter() - th0
    pre_cold = [ev.elapsed_ms(4 * i, 4 * i + 1) for i in range(args.steps)]
    post_cold = [ev.elapsed_ms(4 * i + 2, 4 * i + 3) for i in range(args.steps)]
    ev.destroy()
    pre_ms, post_ms = float(np.mean(pre_cold)), float(np.mean(post_cold))
    ms_per_step = pre_ms + post_ms

    # Back to back: the same K steps with nothing between the launches (post
    # then reads the residual pre left partly in the memory-side cache)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_pre(i % nsets)
        run_post(i % nsets)
    torch.cuda.synchronize()
    ms_per_step_b2b = (time.perf_counter() - t0) * 1e3 / args.steps
    # ... and with an event around every call, for the per-kernel durations
    ev = HipEvents(stream.cuda_stream, 3 * args.steps)
    torch.cuda.synchronize()
    for i in range(args.steps):
        ev.record(3 * i)
        run_pre(i % nsets)
        ev.record(3 * i + 1)
        run_post(i % nsets)
        ev.record(3 * i + 2)
    torch.cuda.synchronize()
    pre_ms_b2b = sum(ev.elapsed_ms(3 * i, 3 * i + 1) for i in range(args.steps)) / args.steps
    post_ms_b2b = sum(ev.elapsed_ms(3 * i + 1, 3 * i + 2) for i in range(args.steps)) / args.steps
    ev.destroy()

    # The layer boundary (mhc_post of one layer, then the next layer's mhc_pre)
    # as one call, on the same buffer sets: the post and comb each set's pre
    # wrote stand for the finished layer's, fn for the next layer's.
    default_wl = args.workload == W.THROUGHPUT_WORKLOAD and spec.n_splits == W.spec(args.workload).n_splits
    for b in sets:
        b["post_next"] = torch.empty_like(b["post"])
        b["comb_next"] = torch.empty_like(b["comb"])

    prep_boundary = [mhc.mhc_post_pre(b["h"], b["residual"], b["post"], b["comb"], fn, hc, bias,
                                      sinkhorn_repeat=spec.sinkhorn_repeat, eps=spec.eps, n_splits=spec.n_splits,
                                      out=b["out"], post_next=b["post_next"], comb_next=b["comb_next"], y=b["y"],
                                      workspace=ws, stream=stream, prepare=True) for b in sets]

    def run_boundary(k):
        prep_boundary[k]()

    for i in range(args.warmup):
        run_boundary(i % nsets)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    for i in range(args.steps):
        run_boundary(i % nsets)
    torch.cuda.synchronize()
    us_b = (time.perf_counter() - t3) * 1e6 / args.steps
    bb = boundary_bytes(T, n, D, e)
    one = bool(mhc.mhc_post_pre_fused(T, n, D, spec.n_splits, 0 if spec.dtype == "bf16" else 1))
    boundary = {"call": "mhc_post_pre", "one_launch": one,
                "traffic": stored_traffic("boundary") if default_wl and one else None,
                "us_per_call": us_b, "tokens_per_s": T / (us_b * 1e-6), "algorithmic_bytes": bb,
                "gbps": bb / (us_b * 1e-6) / 1e9, "frac_of_peak": bb / (us_b * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                "vs_pre_plus_post_step": ms_per_step * 1e3 / us_b}

    # Decode sizes: the layer boundaries of a 16-layer stretch captured in one
    # HIP graph (a decode step's launches as one replay), per boundary call.
    if one and T <= 256 and not args.graph:
        layers = 16
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(layers):
                b = sets[i % nsets]
                mhc.mhc_post_pre(b["h"], b["residual"], b["post"], b["comb"], fn, hc, bias,
                                 sinkhorn_repeat=spec.sinkhorn_repeat, eps=spec.eps, n_splits=spec.n_splits,
                                 out=b["out"], post_next=b["post_next"], comb_next=b["comb_next"], y=b["y"],
                                 workspace=ws, stream=torch.cuda.current_stream(dev))
        for _ in range(3):
            gr.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // layers)
        t4 = time.perf_counter()
        for _ in range(reps):
            gr.replay()
        torch.cuda.synchronize()
        boundary["graph_of_16_us_per_call"] = (time.perf_counter() - t4) * 1e6 / (reps * layers)
        del gr

    # the boundary call alone after the same sweep
    ev = HipEvents(stream.cuda_stream, 2 * args.steps)
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush.max()
        ev.record(2 * i)
        run_boundary(i % nsets)
        ev.record(2 * i + 1)
    torch.cuda.synchronize()
    cb = float(np.mean([ev.elapsed_ms(2 * i, 2 * i + 1) * 1e3 for i in range(args.steps)]))
    ev.destroy()
    del flush
    boundary["us_per_call_back_to_back"] = us_b
    boundary.update({"us_per_call": cb, "tokens_per_s": T / (cb * 1e-6), "gbps": bb / (cb * 1e-6) / 1e9,
                     "frac_of_peak": bb / (cb * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                     "vs_pre_plus_post_step": ms_per_step * 1e3 / cb})

    # practical ceiling: a 1 GiB device-to-device copy kernel on the same stream
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    bp, bq = pre_bytes(T, n, D, e), tail_bytes(T, n, D, e)
    step_gbps = (bp + bq) / (ms_per_step * 1e-3) / 1e9
    post_gbps = bq / (post_ms * 1e-3) / 1e9
    pre_gbps = bp / (pre_ms * 1e-3) / 1e9
    b2b_gbps = (bp + bq) / (ms_per_step_b2b * 1e-3) / 1e9
    pre_kernel = ("pre_resident_kernel (mhc_pre, one launch)" if single
                  else "mhc_pre (fn pack + split-K GEMM + epilogue launches)")
    tail_kernel = "post_combine_norm_kernel" if fused_tail else "post_kernel (mhc_post)"
    result = {
        "metric": METRIC,
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": spec.name, "T": T, "n": n, "D": D, "n_splits": S,
                   "path": "single-pass" if single else "two-pass",
                   "sinkhorn_repeat": spec.sinkhorn_repeat, "buffer_sets": nsets,
                   "launch": "hip-graph replay per call" if args.graph else "direct (C-ABI call per launch)",
                   "timing": "each call after a 1 GiB read sweep (outside the events); ms_per_step = mean pre + "
                             "mean post call"},
        "hbm_gbps": step_gbps,
        "hbm_frac_of_peak": step_gbps / PEAK_HBM_GBPS,
        "algorithmic_bytes_per_step": bp + bq,
        "pre_us": pre_ms * 1e3,
        "post_us": post_ms * 1e3,
        "pre_us_median": float(np.median(pre_cold)) * 1e3,
        "post_us_median": float(np.median(post_cold)) * 1e3,
        "pre_gbps": pre_gbps,
        "post_gbps": post_gbps,
        "headline_wall_s": headline_wall_s,
        "back_to_back": {"ms_per_step": ms_per_step_b2b, "tokens_per_s": T / (ms_per_step_b2b * 1e-3),
                         "hbm_gbps": b2b_gbps, "pre_us": pre_ms_b2b * 1e3, "post_us": post_ms_b2b * 1e3,
                         "note": "no sweep between calls: post reads residual lines pre left in the memory-side "
                                 "cache"},
        "copy_gbps_1GiB": copy_gbps,
        "hbm_frac_of_copy": step_gbps / copy_gbps,
        "tail": "mhc_post_combine_norm (fused, writes out too)" if fused_tail else "mhc_post",
        "boundary": boundary,
        # the pre call is the longer of the two
        "roofline": {"kernel": pre_kernel, "bound": "hbm", "achieved": pre_gbps,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": pre_gbps / PEAK_HBM_GBPS,
                     "traffic": stored_traffic("pre") if default_wl and single else None,
                     "algorithmic_bytes_per_launch": bp},
        "roofline_tail": {"kernel": tail_kernel, "bound": "hbm", "achieved": post_gbps,
                          "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": post_gbps / PEAK_HBM_GBPS,
                          "traffic": stored_traffic("post") if default_wl and not fused_tail else None,
                          "algorithmic_bytes_per_launch": bq},
        "inputs_sha256": x.checksums(),
        "host": host_info(),
        "revision": revision_info(),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill-d7168")
    ap.add_argument("--n-splits", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets the steps rotate over (0: by size)")
    ap.add_argument("--graph", action="store_true",
                    help="capture every call in a HIP graph and replay it (measured slower than direct launches here)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--summarize-rocprof", metavar="DIR")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic profiles from a FETCH_SIZE and a WRITE_SIZE rocprofv3 pass")
    ap.add_argument("--traffic-command", action="append", default=[],
                    help="a line of the command that made the counter passes (recorded in the profile)")
    args = ap.parse_args()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof, args.warmup, args.steps)
        return
    if args.write_traffic:
        write_traffic(*args.write_traffic, args.traffic_command)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (every token is independent, so "
              "data parallelism over tokens needs no communication and N GPUs would each run this step on "
              "their own tokens). Run with --gpus 1.", file=sys.stderr)
        raise SystemExit(2)
    run(args)


if __name__ == "__main__":
    main()
