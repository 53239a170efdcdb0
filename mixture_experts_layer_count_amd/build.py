"""Build libmoe.so (gfx950) in-tree with hipcc, and its bounds-checked debug
twin libmoe_debug.so (every source compiled with -DMOE_BOUNDS_CHECK).

Usage: python -m mixture_experts_layer_count_amd.build  [--jobs N] [--release-only]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmoe.so")
OUT_DEBUG = os.path.join(PKG, "libmoe_debug.so")
BUILD_DIR = os.path.join(PKG, "_build")
BUILD_DIR_DEBUG = os.path.join(PKG, "_build_debug")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-variable", "-Wno-unused-function",
    # packed-FP32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _file_flags(src: str) -> list[str]:
    """Extra flags a source asks for on a `// build-flags: ...` line in its
    header comment."""
    with open(src, encoding="utf-8") as fh:
        for _ in range(12):
            line = fh.readline()
            if line.startswith("// build-flags:"):
                return line.split(":", 1)[1].split()
    return []


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(BUILD_DIR_DEBUG if debug else BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *(["-DMOE_BOUNDS_CHECK"] if debug else []), *_file_flags(src), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _build_one(jobs: int, debug: bool, verbose: bool) -> str:
    out = OUT_DEBUG if debug else OUT
    os.makedirs(BUILD_DIR_DEBUG if debug else BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda src: _compile(src, debug), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build(jobs: int = 8, verbose: bool = False, debug: bool = True) -> str:
    """Compile every HIP source under csrc/ and link libmoe.so, then (unless
    debug=False) the bounds-checked libmoe_debug.so. Always rebuilds."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    out = _build_one(jobs, False, verbose)
    if debug:
        _build_one(jobs, True, verbose)
    return out


def clean() -> None:
    shutil.rmtree(BUILD_DIR, ignore_errors=True)
    shutil.rmtree(BUILD_DIR_DEBUG, ignore_errors=True)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--release-only", action="store_true", help="skip the bounds-checked libmoe_debug.so")
    a = ap.parse_args()
    try:
        build(a.jobs, verbose=True, debug=not a.release_only)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
