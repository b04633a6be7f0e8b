"""Compile the HIP sources into the in-tree shared library ``libmhc.so`` (gfx950).

Usage: ``python -m mhc_hyper_connection_pre_amd.build`` (or ``build_library()``).
Each source is compiled to an object in parallel, then linked. hipcc
cross-compiles for gfx950 without a GPU present.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmhc.so")
OBJDIR = os.path.join(ROOT, "_build")

SOURCES = ["mhc_api.cpp", "mhc_tile_table.cpp", "mhc_pre.hip", "mhc_pre_resident.hip", "mhc_post.hip",
           "mhc_static.hip"]
ARCH = os.environ.get("MHC_OFFLOAD_ARCH", "gfx950")

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions: hipcc must not form v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libmhc.so")
    return path


def build_library(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link ``libmhc.so``; returns its path. Always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [cc, *COMMON_FLAGS, f"--offload-arch={ARCH}", "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd = [cc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out, flush=True)
    if failed:
        msg = "\n".join(f"--- {s}\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp, LIB)
    _write_revision()
    return LIB


REVISION_FILE = os.path.join(PKG, "libmhc.revision")


def _write_revision() -> None:
    """Record beside the library the git revision of the tree it was built from (and whether the tree had
    uncommitted changes), for copies of the tree that travel without their history."""
    rev, dirty = None, None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        if r.returncode == 0:
            rev = r.stdout.strip() or None
            d = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--untracked-files=no"],
                               capture_output=True, text=True, timeout=10)
            dirty = bool(d.stdout.strip()) if d.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        pass
    with open(REVISION_FILE, "w") as f:
        f.write(f"git: {rev}\ndirty: {dirty}\n")


HOST_SOURCES = [s for s in SOURCES if s.endswith(".cpp")]
HOSTSAN_LIB = os.path.join(OBJDIR, "libmhc_hostsan.so")


def build_hostsan_library(verbose: bool = False) -> str:
    """A build of the C ABI whose host-only sources (argument checks, plans,
    the tile table) carry AddressSanitizer and UndefinedBehaviorSanitizer,
    linked with the kernels' objects of the last ``build_library()`` (device
    code is not instrumented). Loading it needs the sanitizer runtime first in
    the process (LD_PRELOAD of ``sanitizer_runtime()``). Returns its path."""
    cc = hipcc()
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".hostsan.o")
        objs.append(obj)
        cmd = [cc, "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"-I{INCLUDE}",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=undefined", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}")
    for src in SOURCES:
        if not src.endswith(".cpp"):
            obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
            if not os.path.exists(obj):
                raise RuntimeError(f"{obj} is missing; run build_library() first")
            objs.append(obj)
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", HOSTSAN_LIB]
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    return HOSTSAN_LIB


def sanitizer_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of the ROCm compiler."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return out.stdout.strip()


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
