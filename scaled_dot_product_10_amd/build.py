"""Build libattn.so in-tree with hipcc for gfx950.

    python -m scaled_dot_product_10_amd.build [--verbose]

Each HIP source compiles to an object under ``_build/`` (in parallel), then
one link step writes ``scaled_dot_product_10_amd/libattn.so``.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = ROOT / "_build"
LIB = PKG / "libattn.so"

SOURCES = ["attn_api.hip", "fwd_bf16.hip", "fwd_f32.hip", "unfused.hip", "bwd_bf16.hip", "splitkv_bf16.hip", "fwd_fp8.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-FP32 instructions: hipcc forms them from plain float code otherwise
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


# The fused kernels' inputs are finite by contract and their masks use -inf
# only, never NaN: without NaN semantics fmaxf maps straight to v_max/v_max3
# (4.6% faster for the fp8 kernel).
PER_FILE_FLAGS = {"fwd_bf16.hip": ["-fno-honor-nans"], "fwd_fp8.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and Path(c).exists():
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libattn)")


def build(verbose: bool = False, extra: list[str] | None = None) -> Path:
    cc = hipcc()
    BUILD.mkdir(exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = BUILD / (Path(src).stem + ".o")
        objs.append(obj)
        cmd = [cc, *FLAGS, *PER_FILE_FLAGS.get(src, []), *(extra or []), "-c", str(CSRC / src), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        # hipcc's host pass does not know the packed-fp32 feature flag; that warning is expected
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    tmp = LIB.with_name(LIB.name + f".tmp{os.getpid()}")
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args()
    print(build(verbose=a.verbose))
