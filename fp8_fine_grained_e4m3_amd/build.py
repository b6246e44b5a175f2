"""Build libdg.so (the C-ABI GEMM library) for gfx950 with hipcc, in-tree.

Usage: python -m fp8_fine_grained_e4m3_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdg.so")
SOURCES = ["dg_api.cpp", "nt_kernel.hip", "tn_kernel.hip", "cast_kernel.hip", "mqa_kernel.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # Never emit packed fp32 VALU ops (v_pk_fma_f32 and friends).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-early-inline-all=true",
]


def build(verbose: bool = False) -> str:
    """Compile every source into libdg.so next to this file; returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libdg.so")
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    os.replace(tmp, LIB)
    return LIB


def resource_usage() -> str:
    """Per-kernel VGPR/SGPR/spill/LDS report of the device code (compile only)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES if s.endswith(".hip")]
    out = []
    for s in srcs:
        cmd = [HIPCC] + [f for f in FLAGS if f not in ("-shared",)] + [
            "--cuda-device-only", "-c", "-Rpass-analysis=kernel-resource-usage", s, "-o",
            os.devnull]
        res = subprocess.run(cmd, capture_output=True, text=True)
        out.append(res.stderr)
    return "\n".join(out)


if __name__ == "__main__":
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        sys.exit(f"hipcc not found at {HIPCC}")
    print(build(verbose=True))
    if "--usage" in sys.argv:
        print(resource_usage())
