"""Tile tuner: time every tiling the library builds for a shape and write the
fastest into the library's tile table.

The split-K pre GEMM is tiled over the hidden axis with a block size picked per
hidden size ([P1] "[sglang] AMD ROCm DeepSeek-V4 performance optimisation:
Aiter MHC kernel integration analysis", section 3, TileLang kernel tuning).
Here the choices are the single-pass kernel's slice count S (n_splits = -S,
D = 32 * cps * S) together with its instance (the workgroup's waves in step,
or one pipeline per wave; chosen through MHC_STAGGER while timing), and the
two-pass path's split count (n_splits = S > 0). For
every (op, n, D, dtype) and every token count T of a sweep, each candidate is
timed call by call, each call after a read of a 1 GiB buffer (so neither L2
nor the 256 MB Infinity Cache holds its inputs, as between a layer's calls in
a model and as bench.py times them), between two HIP events on the launch
stream, over input sets it rotates through, in several rounds that visit the
candidates in turn; a candidate's time is its median over the rounds
(--back-to-back times back-to-back calls instead). The fastest becomes the table
entry for the token range around T (range ends at the geometric means of
neighbouring sweep points); the library's own single-pass tiling is kept when
it is within 3 % of the fastest, so noise does not flip the choice.

Usage, on the GPU, then rebuild the library:

    python -m mhc_hyper_connection_pre_amd.tune \\
        --json mhc_hyper_connection_pre_amd/tile_table.json \\
        --cpp mhc_hyper_connection_pre_amd/csrc/mhc_tile_table.cpp

``--json`` keeps every measurement; ``--cpp`` is the table compiled into the
library (entries are used by ``n_splits = 0`` when they cover a call and are
valid for it).
"""

from __future__ import annotations

import argparse
import datetime
import json
import math
import os
import statistics
import sys

import mhc_hyper_connection_pre_amd as mhc

DEFAULT_SHAPES = ["2,4096", "2,7168", "3,3072", "4,4096", "4,5120", "4,6144", "4,7168", "8,4096", "8,7168"]
DEFAULT_TOKENS = [16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384]
TWO_PASS_SPLITS = [1, 2, 4, 8, 16, 32, 64]
KEEP_LIBRARY_WITHIN = 1.03
T_MAX = 2 ** 31 - 1


def candidates(op: str, T: int, n: int, D: int, dt: int) -> list[tuple[int, int]]:
    """(n_splits, instance) pairs the library accepts for the shape: each single-pass slice count with the
    waves in step (0) and with one pipeline per wave (1), then the two-pass split counts (instance -1)."""
    L = mhc.lib()
    out = []
    for S in range(2, 257):
        if L.mhc_pre_splits(T, n, D, -S, dt) != S:
            continue
        if op == "boundary" and L.mhc_post_pre_fused(T, n, D, -S, dt) != 1:
            continue
        out += [(-S, 0), (-S, 1)]
    for S in TWO_PASS_SPLITS:
        if L.mhc_pre_splits(T, n, D, S, dt) == S:
            out.append((S, -1))
    return out


def key(c: tuple[int, int]) -> str:
    """Record key of a candidate: '-32/1' (single-pass, instance) or '8' (two-pass)."""
    return f"{c[0]}/{c[1]}" if c[0] < 0 else str(c[0])


_CALLER_STAGGER = os.environ.get("MHC_STAGGER")


def _instance(c: tuple[int, int]) -> None:
    """Select the single-pass instance for the next calls (MHC_STAGGER is read at each launch); instance -1
    restores the caller's setting."""
    if c[1] >= 0:
        os.environ["MHC_STAGGER"] = str(c[1])
    elif _CALLER_STAGGER is None:
        os.environ.pop("MHC_STAGGER", None)
    else:
        os.environ["MHC_STAGGER"] = _CALLER_STAGGER


def set_count(T: int, n: int, D: int, elem: int) -> int:
    """Input sets to rotate over: between two uses of one set the others move twice the 256 MB Infinity Cache."""
    per_set = T * (2 * n + 2) * D * elem   # residual, out, h, y
    return max(2, min(8, -(-2 * 256 * 10 ** 6 // max(per_set, 1)) + 1))


class _Inputs:
    """Device input sets (and outputs) of one shape, random values of the workloads' scale."""

    def __init__(self, torch, T: int, n: int, D: int, dtype, seed: int):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        N = n * (n + 2)
        dev = "cuda"
        self.sets = []
        for _ in range(set_count(T, n, D, 2 if dtype == torch.bfloat16 else 4)):
            s = {
                "residual": torch.randn((T, n, D), generator=g, device=dev).to(dtype),
                "h": torch.randn((T, D), generator=g, device=dev).to(dtype),
                "fn": torch.randn((n * D, N), generator=g, device=dev) * 0.01,
                "hc_scale": torch.ones(3, device=dev),
                "bias": torch.randn(N, generator=g, device=dev) * 0.1,
                "post_in": torch.rand((T, n), generator=g, device=dev),
                "comb_in": torch.rand((T, n, n), generator=g, device=dev) / n,
                "post": torch.empty((T, n), device=dev),
                "comb": torch.empty((T, n, n), device=dev),
                "y": torch.empty((T, D), dtype=dtype, device=dev),
                "out": torch.empty((T, n, D), dtype=dtype, device=dev),
            }
            self.sets.append(s)


def _call(op: str, s: dict, n_splits: int, ws) -> None:
    if op == "pre":
        mhc.mhc_pre(s["residual"], s["fn"], s["hc_scale"], s["bias"], n_splits=n_splits, post=s["post"],
                    comb=s["comb"], y=s["y"], workspace=ws)
    else:
        mhc.mhc_post_pre(s["h"], s["residual"], s["post_in"], s["comb_in"], s["fn"], s["hc_scale"], s["bias"],
                         n_splits=n_splits, out=s["out"], post_next=s["post"], comb_next=s["comb"], y=s["y"],
                         workspace=ws)


def time_candidate(torch, op: str, inputs: _Inputs, n_splits: int, ws, iters: int, warmup: int,
                   sweep=None) -> float:
    """Microseconds per call, after `warmup` calls. Without `sweep`: `iters` back-to-back calls between two
    events. With `sweep` (a device buffer of 1 GiB): each call alone between two events after a read of the
    whole buffer, which leaves neither L2 nor the memory-side cache holding its inputs (as between a layer's
    calls in a model, and as bench.py times them); the median of `iters` calls."""
    k = len(inputs.sets)
    for i in range(warmup):
        _call(op, inputs.sets[i % k], n_splits, ws)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if sweep is None:
        e0.record()
        for i in range(iters):
            _call(op, inputs.sets[i % k], n_splits, ws)
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / iters
    ts = []
    for i in range(iters):
        sweep.max()
        e0.record()
        _call(op, inputs.sets[i % k], n_splits, ws)
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1000.0)
    return statistics.median(ts)


def pick(times: dict, library=None):
    best = min(times, key=times.get)
    if library is not None and library in times and times[library] <= times[best] * KEEP_LIBRARY_WITHIN:
        return library
    return best


def ranges(points: list[tuple]) -> list[tuple]:
    """[(T, choice...)] sorted by T -> [(T_lo, T_hi, choice...)], neighbours with one choice merged."""
    out = []
    for i, (T, *choice) in enumerate(points):
        lo = 1 if i == 0 else int(math.sqrt(points[i - 1][0] * T)) + 1
        hi = T_MAX if i == len(points) - 1 else int(math.sqrt(T * points[i + 1][0]))
        if out and list(out[-1][2:]) == choice:
            out[-1] = (out[-1][0], hi, *choice)
        else:
            out.append((lo, hi, *choice))
    return out


def write_cpp(path: str, entries: list[dict], device: str, stamp: str) -> None:
    lines = []
    for e in entries:
        for lo, hi, ns, st in ranges([(p["T"], p["best"], p["stagger"]) for p in e["points"]]):
            lines.append(f"    {{{0 if e['op'] == 'pre' else 1}, {e['n']}, {e['D']}, {e['dt']}, {lo}, {hi}, {ns}, {st}}},")
    body = "\n".join(lines)
    text = f"""// Tile table: the n_splits (and for the single-pass kernel its instance) that
// measured fastest for listed shapes (op, n, D, dtype, token range). Written
// by mhc_hyper_connection_pre_amd/tune.py; the library's choice (n_splits = 0)
// takes an entry that covers the call and is valid for it, and its heuristic
// otherwise.
// Measured on {device} ({stamp}).

#include "mhc_internal.h"

namespace mhc {{
namespace {{

struct TileEntry {{
  int op;               // 0 = mhc_pre, 1 = mhc_post_pre
  int n;
  int64_t D;
  int dt;               // mhc_dtype
  int64_t T_lo, T_hi;   // token counts the entry covers, inclusive
  int n_splits;         // -S: single-pass with S slices; S > 0: two-pass with S splits
  int stagger;          // single-pass instance: 0 waves in step, 1 one pipeline per wave; -1 the library's rule
}};

constexpr TileEntry kTable[] = {{
{body}
    {{-1, 0, 0, 0, 0, 0, 0, -1}},   // end
}};

}}  // namespace

int tuned_splits(int64_t T, int n, int64_t D, mhc_dtype dt, bool boundary, int* stagger) {{
  if (stagger) *stagger = -1;
  for (const TileEntry& e : kTable) {{
    if (e.op == (boundary ? 1 : 0) && e.n == n && e.D == D && e.dt == (int)dt && T >= e.T_lo && T <= e.T_hi) {{
      if (stagger) *stagger = e.stagger;
      return e.n_splits;
    }}
  }}
  return 0;
}}

}}  // namespace mhc
"""
    with open(path, "w") as f:
        f.write(text)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--shapes", nargs="*", default=DEFAULT_SHAPES, help="n,D[,dtype] (dtype bf16 or f32)")
    ap.add_argument("--tokens", nargs="*", type=int, default=DEFAULT_TOKENS)
    ap.add_argument("--ops", nargs="*", default=["pre", "boundary"], choices=["pre", "boundary"])
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--back-to-back", action="store_true",
                    help="time back-to-back calls instead of each call after a 1 GiB read sweep")
    ap.add_argument("--json", default=None, help="write every measurement here")
    ap.add_argument("--cpp", default=None, help="write the library's tile table source here")
    args = ap.parse_args(argv)

    import torch
    if not torch.cuda.is_available():
        print("tune: no GPU visible", file=sys.stderr)
        return 2
    props = torch.cuda.get_device_properties(0)
    device = f"{props.name} ({props.gcnArchName.split(':')[0]}, {props.multi_processor_count} CUs)"
    stamp = datetime.datetime.now(datetime.timezone.utc).strftime("%Y-%m-%d %H:%M UTC")
    L = mhc.lib()
    sweep = None if args.back_to_back else torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    entries = []
    for shape in args.shapes:
        parts = shape.split(",")
        n, D = int(parts[0]), int(parts[1])
        dname = parts[2] if len(parts) > 2 else "bf16"
        dt = mhc.MHC_BF16 if dname == "bf16" else mhc.MHC_F32
        dtype = torch.bfloat16 if dname == "bf16" else torch.float32
        for op in args.ops:
            e = {"op": op, "n": n, "D": D, "dtype": dname, "dt": dt, "points": []}
            for T in sorted(args.tokens):
                cands = candidates(op, T, n, D, dt)
                if not cands:
                    continue
                inputs = _Inputs(torch, T, n, D, dtype, seed=T * 31 + D)
                need = max(L.mhc_pre_workspace_bytes(T, n, D, c[0], dt) for c in cands)
                ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
                ws[:256].zero_()
                runs = {c: [] for c in cands}
                for _ in range(args.rounds):
                    for c in cands:
                        _instance(c)
                        runs[c].append(time_candidate(torch, op, inputs, c[0], ws, args.iters, args.warmup, sweep))
                _instance((0, -1))
                times = {c: statistics.median(v) for c, v in runs.items()}
                lib_sp = L.mhc_pre_splits(T, n, D, -1, dt)
                # the library's own single-pass slicing, in the faster of its two instances
                lib = [c for c in times if c[0] == -lib_sp] if lib_sp > 0 else []
                library = min(lib, key=times.get) if lib else None
                best = pick(times, library)
                e["points"].append({"T": T, "best": best[0], "stagger": best[1],
                                    "library_single_pass": None if library is None else key(library),
                                    "us": {key(c): round(v, 2) for c, v in times.items()}})
                print(f"{op:8s} n={n} D={D} {dname} T={T:6d}: best {key(best):>8s} "
                      f"({times[best]:.1f} us; library single-pass "
                      f"{'-' if library is None else f'{key(library)} {times[library]:.1f} us'})", flush=True)
                del inputs, ws
                torch.cuda.empty_cache()
            entries.append(e)
    if args.json:
        with open(args.json, "w") as f:
            json.dump({"device": device, "measured": stamp, "iters": args.iters, "warmup": args.warmup,
                       "rounds": args.rounds, "timing": "back to back" if args.back_to_back else
                       "each call after a 1 GiB read sweep", "entries": entries}, f, indent=1)
    if args.cpp:
        write_cpp(args.cpp, entries, device, stamp)
    return 0


if __name__ == "__main__":
    sys.exit(main())
