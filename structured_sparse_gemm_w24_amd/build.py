"""Builds libssg.so in-tree: host C++ with g++, HIP sources with hipcc for gfx950.

    python -m structured_sparse_gemm_w24_amd.build [--jobs N] [--save-temps]

Every call recompiles.  Objects go to ``_build/`` at the repository root; the
library lands next to this file.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libssg.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")

# -packed-fp32-ops: keep the compiler from forming packed fp32 arithmetic.
# -ffp-contract=off: the int8 epilogues compute float(acc) * scale, then
# + bias, each rounded on its own; HIP's __fmul_rn / __fadd_rn are plain
# operators, which the default contraction may fuse into one multiply-add
# (one rounding), changing results at fp16 / int8 rounding boundaries.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
             "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra"]

HOST_SOURCES = ["status.cpp", "pack.cpp"]
HIP_SOURCES = ["api.hip", "kernels/gemm.hip", "kernels/splitk.hip", "kernels/tw_gemm.hip",
               "kernels/tw_gemm_i8.hip", "kernels/transpose.hip"]


def _obj(src):
    return os.path.join(BUILD, src.replace("/", "_") + ".o")


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + p.stdout + p.stderr)
    return p.stderr


def build(jobs=8, save_temps=False, verbose=False):
    """Compile every source and link libssg.so; returns the library path."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    cmds = []
    for s in HOST_SOURCES:
        cmds.append([CXX, *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", _obj(s)])
    for s in HIP_SOURCES:
        extra = ["-save-temps=obj"] if save_temps else []
        cmds.append([HIPCC, *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, s), "-o", _obj(s)])
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for err in ex.map(_run, cmds):
            if verbose and err.strip():
                sys.stderr.write(err)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp,
          *[_obj(s) for s in HOST_SOURCES + HIP_SOURCES]])
    os.replace(tmp, LIB)
    build_vendor()
    build_peak()
    return LIB


VENDOR_LIB = os.path.join(PKG, "libssg_vendor.so")
VENDOR_HEADER = "/opt/rocm/include/hipsparselt/hipsparselt.h"


def build_vendor():
    """The bench's vendor 2:4 baseline (hipSPARSELt), when its headers are
    installed; a separate library that libssg never loads.  A failure here is
    reported and leaves the product build alone (the bench then skips the
    vendor columns)."""
    if not os.path.exists(VENDOR_HEADER):
        return None
    tmp = VENDOR_LIB + ".tmp"
    try:
        _run([HIPCC, "--offload-arch=" + ARCH, "-O2", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
              "-Wno-unused-command-line-argument", os.path.join(CSRC, "vendor", "hipsparselt_ref.cpp"),
              "-o", tmp, "-lhipsparselt"])
    except RuntimeError as e:
        print(f"note: vendor baseline library not built ({str(e).splitlines()[0]})", file=sys.stderr)
        return None
    os.replace(tmp, VENDOR_LIB)
    return VENDOR_LIB


PEAK_LIB = os.path.join(PKG, "libssg_peak.so")


def build_peak():
    """The bench's matrix-core rate probe (a separate library that libssg never
    loads).  A failure here is reported and leaves the product build alone (the
    bench then reports no measured MFMA peak)."""
    tmp = PEAK_LIB + ".tmp"
    try:
        _run([HIPCC, *HIP_FLAGS, "-shared", os.path.join(CSRC, "bench", "mfma_peak.hip"), "-o", tmp])
    except RuntimeError as e:
        print(f"note: matrix-core rate probe not built ({str(e).splitlines()[0]})", file=sys.stderr)
        return None
    os.replace(tmp, PEAK_LIB)
    return PEAK_LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--save-temps", action="store_true", help="keep device assembly in _build/")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.save_temps, a.verbose))


if __name__ == "__main__":
    main()
