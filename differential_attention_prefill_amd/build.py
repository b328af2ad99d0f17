"""Build libdiffattn.so: the HIP kernels and the C ABI, for gfx950 only.

Every source is compiled with hipcc for --offload-arch=gfx950, packed fp32
vector instructions disabled, into objects under _build/, then linked
in-tree next to this file so the library travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdiffattn.so")

SOURCES = ["api.cpp", "shapes.cpp", "lambda.hip", "prefill_f32.hip", "prefill_pp.hip", "combine.hip",
           "decode.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


# The fused prefill runs with the IEEE mode bit off (its row maxima then need
# no NaN-quieting instructions); scores there are never NaN.
EXTRA_FLAGS = {"prefill_pp.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + EXTRA_FLAGS.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s%s" % (src, r.stdout, r.stderr))
    return obj


def build(jobs: int = 8) -> str:
    """Compile every source and link libdiffattn.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
