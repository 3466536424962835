"""Build libfp4mx.so (HIP, gfx950 only) in-tree with hipcc.

Usage: ``python -m fp4_microscaled_quantized_amd.build`` or ``build_library()``.
The library is written next to this file; it is not installed anywhere.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfp4mx.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["quant_mx.hip", "gemm_mx.hip", "nvfp4.hip", "msedn.hip", "quest.hip", "abi.hip"]
# measurement aid (the benchmark's sustained-MFMA roofline), its own library
PROBE_SOURCES = ["probe_mfma.hip"]
PROBE_LIB = os.path.join(PKG, "libfp4mx_probe.so")
# measurement and cross-check aid: hipBLASLt's MXFP4 GEMM behind a C ABI (the
# benchmark times it beside fp4mx_gemm; a GPU test compares the outputs)
VENDOR_SOURCES = ["vendor_gemm.cpp"]
VENDOR_LIB = os.path.join(PKG, "libfp4mx_vendor.so")
VENDOR_LINK = ["-L/opt/rocm/lib", "-lhipblaslt"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # exact IEEE fp32 semantics: no FMA contraction, no denormal flushing,
    # correctly rounded fp32 division (the NVFP4 quantizer divides)
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE,
    "-I" + CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs, lib, extra=()):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + list(extra)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES + VENDOR_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    n0, n1 = len(SOURCES), len(SOURCES) + len(PROBE_SOURCES)
    _link(objs[:n0], LIB)
    _link(objs[n0:n1], PROBE_LIB)
    _link(objs[n1:], VENDOR_LIB, VENDOR_LINK)
    if verbose:
        print("built", LIB, PROBE_LIB, "and", VENDOR_LIB)
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
