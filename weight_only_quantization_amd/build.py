"""Build libhqq.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m weight_only_quantization_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhqq.so")
PROBE_LIB = os.path.join(HERE, "libhqq_probe.so")
OBJDIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -ffp-contract=off: the quantizer's fp64 arithmetic must round each written operation
# (fma only where the source says fma).  Packed fp32 instructions are disabled.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I" + os.path.join(HERE, "..", "include")]

SOURCES = ["hqq_api.hip", "hqq_quant.hip", "hqq_dequant.hip", "hqq_gemv.hip", "hqq_gemv_ext.hip", "hqq_gemv_dq.hip", "hqq_gemm.hip"]
# HBM probes of known byte counts (measurement only), a library of their own
PROBE_SOURCES = ["hqq_probe.hip"]

# The split GEMM keeps its 128 MFMA accumulators per lane in ordinary VGPRs: with the default
# (accumulation-register) form the register allocator does not tie each MFMA's result to its
# accumulator input and copies accumulators between register files around most MFMAs.
EXTRA = {"hqq_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp, *objs])
    os.replace(tmp, lib)


def build(jobs: int = 4) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    a = ap.parse_args()
    print(build(a.jobs))
