"""Build libmoe_offload.so for gfx950 in-tree (hipcc; one object per source, then link)."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmoe_offload.so")
BUILD = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "k_route.hip", "k_gemv.hip", "k_gemv_gateup_bf16.hip", "k_gemv_gateup_f32.hip",
           "k_gemv_down_bf16.hip", "k_gemv_down_f32.hip", "k_gemm.hip", "k_stage.hip", "k_util.hip", "k_gemv_lowbit_gateup.hip",
           "k_gemv_lowbit_down.hip", "host_logic.cpp", "host_ffn.cpp"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
# packed fp32 math is kept out of every kernel
HIP_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# the host expert FFN is AVX-512 code; the library calls it only where the CPU has AVX-512
HOST_FLAGS = {"host_ffn.cpp": ["-mavx512f", "-mavx512bw", "-mavx512vl", "-mf16c", "-mfma"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC] + HIP_FLAGS + COMMON + ["-c", path, "-o", obj]
    else:
        cmd = ["g++"] + COMMON + ["-Wall", "-c", path, "-o", obj] + HOST_FLAGS.get(src, [])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + ["-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
