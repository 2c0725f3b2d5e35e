"""Build libdwconv.so: the gfx950 HIP kernels and the C ABI in include/dwconv.h.

Every ``csrc/*.hip`` file is compiled with hipcc for gfx950 into an object under
``_build/`` and the objects are linked into ``dynamic_convolution_amd/libdwconv.so``
(in-tree, so it travels with the source tree).  Packed-FP32 VALU instructions are
disabled (``-packed-fp32-ops``): hipcc only forms them by itself from plain float
code, and every kernel here is written with scalar fp32 FMAs.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdwconv.so")
# device-ceiling probes for the benchmark's roofline; not part of the library
PROBE_SRC = os.path.join(PKG, "probe", "dw_probe.hip")
PROBE_LIB = os.path.join(PKG, "libdwprobe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


# Per-source code generation options: the row-streaming 16-bit kernels keep
# their matrix accumulators in ordinary VGPRs (their bookkeeping moves single
# accumulator elements, which the AGPR form turns into register copies).
EXTRA_FLAGS = {
    "dw_largek_roll16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "dw_largek_wroll16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "dw_largek_rollf32.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stdout))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every kernel source for gfx950 and link libdwconv.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stdout)
    os.replace(tmp, LIB)
    build_probe()
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


def build_probe() -> str:
    """Compile the benchmark's device-ceiling probes into libdwprobe.so."""
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + [f for f in FLAGS if not f.startswith("-I")] + ["-shared", "-o", tmp, PROBE_SRC]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (PROBE_SRC, r.stdout))
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
