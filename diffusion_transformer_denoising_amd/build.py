"""Build libdit.so (gfx950) and the synthetic-input generator's C core in-tree.

    python -m diffusion_transformer_denoising_amd.build

Each HIP source is compiled to an object under ``_build/`` in parallel, then
linked into ``diffusion_transformer_denoising_amd/libdit.so``.  Always
recompiles: the build is the "does it build" check.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libdit.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.cpp", "gemm.hip", "attention.hip", "pointwise.hip", "cache.hip"]

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    "-I", INCLUDE, "-I", CSRC,
    # no packed-fp32 VALU instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build_synth() -> str:
    src = os.path.join(ROOT, "synth", "philox_words.c")
    out = os.path.join(ROOT, "synth", "_philox_words.so")
    _run(["gcc", "-O3", "-fopenmp", "-shared", "-fPIC", src, "-o", out, "-lm"])
    return out


def build_lib(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + HIP_FLAGS
        if src.endswith(".cpp"):
            cmd += ["-x", "hip"]
        cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
        out = _run(cmd)
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def build(verbose: bool = False) -> None:
    build_synth()
    build_lib(verbose)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB_PATH)
