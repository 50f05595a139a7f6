"""Build libqmm.so in-tree for gfx950 with hipcc (run: python -m bit_affine_quantized_qmv_amd.build)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqmm.so")
SOURCES = ["decode_b4.hip", "decode_b8.hip", "decode_bn.hip", "decode.cpp", "prefill.hip", "dequant.hip", "quantize.hip", "topk.hip", "noalloc.hip", "dispatch.cpp", "capi.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed float32 instructions stay disabled for every device pass.
COMMON = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    return obj


# Test helper built beside the library: fills and reads back LDS between library kernels.
TEST_HELPER_SRC = os.path.join(ROOT, "tests", "lds_fill.hip")
TEST_HELPER_LIB = os.path.join(ROOT, "tests", "_lds_fill.so")


def build_test_helper(verbose: bool = True) -> str:
    tmp = TEST_HELPER_LIB + ".tmp"
    cmd = [HIPCC] + COMMON + ["-x", "hip", "-shared", TEST_HELPER_SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for the test helper:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, TEST_HELPER_LIB)
    if verbose:
        print("built", TEST_HELPER_LIB)
    return TEST_HELPER_LIB


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    build_test_helper(verbose)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
