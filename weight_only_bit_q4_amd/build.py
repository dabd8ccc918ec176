"""Build the q4lin HIP library (gfx950) in-tree.

``python -m weight_only_bit_q4_amd.build`` compiles every ``csrc/*.hip`` with
hipcc for gfx950 and links ``weight_only_bit_q4_amd/libq4lin.so``, and the
benchmark's ceiling probes (``csrc/probe/*.hip``, not part of the op) into
``weight_only_bit_q4_amd/libq4lin_probe.so``.  Object files go to ``_build/``
at the repository root.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libq4lin.so")
PROBE_LIB = os.path.join(PKG, "libq4lin_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden",
    # torch ships its own HIP runtime (ROCm 7.0) and the process uses that one;
    # code object v5 loads on it and on newer runtimes
    "-mcode-object-version=5",
    # packed FP32 vector instructions stay off in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unknown-warning-option", "-Wno-cuda-compat",
    "-I", os.path.join(ROOT, "include"),
]


# Matrix-core results in ordinary VGPRs for every kernel but the tiled one:
# the small-T kernel scales every group's products with VALU instructions,
# which cannot read accumulator registers; the tiled kernel keeps its
# accumulators in AGPRs, away from its VALU work.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
AGPR_ACC_SOURCES = {"q4lin_tiled.hip"}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    extra = [] if os.path.basename(src) in AGPR_ACC_SOURCES else VGPR_FORM
    cmd = [HIPCC] + CFLAGS + extra + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only target feature; drop that note
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-mcode-object-version=5", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probe_srcs = sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probe_srcs))) as ex:
        objs = list(ex.map(_compile, srcs + probe_srcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print("built", LIB)
        print("built", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
