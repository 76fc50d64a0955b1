"""Build the native libraries in-tree.

  libpa.so       -- the product: host manager + HIP kernels for gfx950
  libpa_host.so  -- the host manager alone, built with g++ (no HIP), for
                    CPU-only tests of the manager

Run ``python -m paged_kv_cache_239_amd.build`` (or call ``build_all()``).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")

LIB = os.path.join(HERE, "libpa.so")
HOST_LIB = os.path.join(HERE, "libpa_host.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU instructions are kept out of every kernel.  Matrix-core
# accumulators stay in ordinary vector registers: left to the compiler's
# heuristic they move between the accumulation and the vector file on every
# step of the attention loops (the online-softmax rescale reads them).
HIP_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-Wall", "-Wno-unused-function"]


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_hip(extra=()):
    srcs = [os.path.join(CSRC, f) for f in ("pa_host.cpp", "pa_attention.hip", "pa_cache.hip")]
    tmp = LIB + ".tmp"
    _run([HIPCC, *HIP_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def build_host(extra=(), out=HOST_LIB):
    cxx = shutil.which("g++") or "g++"
    tmp = out + ".tmp"
    _run([cxx, "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", *extra, "-I", INCLUDE, "-I", CSRC,
          os.path.join(CSRC, "pa_host.cpp"), "-o", tmp])
    os.replace(tmp, out)
    return out


def build_all():
    build_host()
    build_hip()


if __name__ == "__main__":
    build_all()
    sys.exit(0)
