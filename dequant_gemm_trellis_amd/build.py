"""Build libtrellis.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Every HIP translation unit is compiled with packed-FP32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); hipcc's host pass warns
that it does not know the feature, which is harmless. No fast-math: the weight
products must be IEEE float32 multiplies rounded to nearest even.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtrellis.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["gemv.hip", "axis1.hip", "axis0.hip", "layout.hip", "probe.hip", "api.cpp"]
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-command-line-argument"]
DEVICE = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=off"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    lang = (["-x", "hip"] if src.endswith(".hip")
            else ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include")])
    cmd = [_hipcc(), *COMMON, *(DEVICE if src.endswith(".hip") else []), *lang, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
