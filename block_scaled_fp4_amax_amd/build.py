"""Build libfp4.so (the HIP kernels + C ABI) in-tree for gfx950.

Every source is compiled with hipcc for gfx950 with packed fp32 arithmetic
disabled and floating-point contraction off (the quantizer's decisions must be
bit-identical to the fp32 step-by-step definition), then linked into
``block_scaled_fp4_amax_amd/libfp4.so``.

Usage: ``python -m block_scaled_fp4_amax_amd.build`` or ``build()``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG_DIR = Path(__file__).resolve().parent
REPO_DIR = PKG_DIR.parent
CSRC = PKG_DIR / "csrc"
INCLUDE = REPO_DIR / "include"
BUILD_DIR = REPO_DIR / "_build"
LIB_PATH = PKG_DIR / "libfp4.so"

SOURCES = ["fp4_api.cpp", "quantize.hip", "dequantize.hip", "gemm.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", str(INCLUDE),
    "-I", str(CSRC),
]


# Per-source flags. gemm.hip: LLVM's machine-sink pass would move a stage's
# first-half MFMAs past the workgroup barrier into the next block (their
# results are only used there), so the wave would wait at the barrier with its
# matrix core idle; the kernel's order is the intended schedule.
SOURCE_FLAGS = {"gemm.hip": ["-mllvm", "-disable-machine-sink"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the FP4 library needs the ROCm toolchain to build")


def build(verbose: bool = False) -> Path:
    """Compile every source (in parallel) and link libfp4.so. Always rebuilds."""
    hipcc = _hipcc()
    BUILD_DIR.mkdir(exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = BUILD_DIR / (src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), *lang, "-c", str(CSRC / src), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out)
    if failed:
        msg = "\n".join(f"--- {s} ---\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB_PATH.with_suffix(".so.tmp")
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
