"""Ahead-of-time build of libmnb.so for gfx950 with hipcc (no JIT, no torch
extension machinery).  ``python -m block_wise_int4_amd.build`` compiles every
source every time; the library lands in ``block_wise_int4_amd/lib/``."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIB_DIR, "libmnb.so")

SOURCES = ["mnb_api.cpp", "repack.hip", "act_order.hip", "gemv.hip", "gemm_small.hip", "gemm_mfma.hip",
           "noalloc.hip", "f32_split.hip", "gidx.hip",
           "acc4.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]
# device code: gfx950 only; packed fp32 VALU ops disabled
DEVICE_FLAGS = [
    "--offload-arch=" + ARCH, "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
]


# per-source extras: the prefill GEMM keeps its MFMA accumulators in VGPRs, so
# the per-group scaling reads them without v_accvgpr_read copies
EXTRA_FLAGS = {"gemm_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               # the first 16 argument dwords of the fp16 GEMV and the small-M kernel
               # arrive in SGPRs (measured faster; the int8-activation GEMV measured
               # slower with it)
               "gemv.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"],
               "gemm_small.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = ([HIPCC] + COMMON_FLAGS + DEVICE_FLAGS + EXTRA_FLAGS.get(src, []) +
           ["-c", os.path.join(CSRC, src), "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


# bench.py's streaming-read yardstick: a library of its own, outside the
# matmul ABI
YARDSTICK_SRC = "yardstick.hip"
YARDSTICK_LIB = os.path.join(LIB_DIR, "libmnb_yardstick.so")


def _build_yardstick() -> str:
    obj = _compile(YARDSTICK_SRC)
    tmp = YARDSTICK_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, YARDSTICK_LIB)
    return YARDSTICK_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES) + 1, os.cpu_count() or 4)) as ex:
        yard = ex.submit(_build_yardstick)
        objs = list(ex.map(_compile, SOURCES))
        yard.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
