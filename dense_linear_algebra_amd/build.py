"""Build libbatchlu.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m dense_linear_algebra_amd.build [-v] [--incremental] [--resources]

Every HIP source is compiled with IEEE semantics: -ffp-contract=off (no fused
multiply-add except the ones the code spells), no fast-math, and without the
packed-FP32 VALU forms.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbatchlu.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math", "-Wall",
          "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-pragma-unroll-threshold=2000000"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def _deps(src: str, seen=None) -> set:
    """src and every file it includes with #include "..." (transitively)."""
    seen = set() if seen is None else seen
    if src in seen or not os.path.exists(src):
        return seen
    seen.add(src)
    with open(src) as f:
        for line in f:
            m = re.match(r'\s*#\s*include\s+"([^"]+)"', line)
            if m:
                for d in (os.path.dirname(src), CSRC, INCLUDE):
                    cand = os.path.normpath(os.path.join(d, m.group(1)))
                    if os.path.exists(cand):
                        _deps(cand, seen)
                        break
    return seen


def _stale(src: str, obj: str) -> bool:
    """True when obj is missing or older than src or a file it includes."""
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in _deps(src))


def _compile(src: str, verbose: bool, extra=(), incremental=False):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if incremental and not extra and not _stale(src, obj):
        return obj, ""
    cmd = [HIPCC, "-c", src, "-o", obj] + COMMON + list(extra)
    if src.endswith(".hip"):
        cmd += DEVICE
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    with open(obj + ".log", "w") as f:
        f.write(r.stderr)
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj, r.stderr


def build_library(verbose: bool = False, jobs: int | None = None, extra=(), incremental: bool = False) -> str:
    """Compile every source (in parallel) and link libbatchlu.so.  Rebuilds
    every object unless ``incremental``, which recompiles only objects older
    than their source or any header of the package."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = [o for o, _ in ex.map(lambda s: _compile(s, verbose, extra, incremental), srcs)]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    v = "-v" in sys.argv
    extra = ["-Rpass-analysis=kernel-resource-usage"] if "--resources" in sys.argv else []
    print(build_library(verbose=v, extra=extra, incremental="--incremental" in sys.argv))
