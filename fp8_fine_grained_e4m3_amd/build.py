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


# Sources compiled on their own with extra flags, then linked in.  The MQA
# kernel consumes every MFMA result on the VALU at once, so it asks for the
# MFMA form that writes VGPRs (no accumulator-register reads); the GEMM
# kernels keep the default.
SEPARATE = {"mqa_kernel.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
OBJ_DIR = os.path.join(HERE, "_build")


def _run(cmd, verbose, what):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed {what}")


def build(verbose: bool = False) -> str:
    """Compile every source (each to its own object, in parallel) and link
    libdg.so next to this file; returns its path."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(OBJ_DIR, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + compile_flags + SEPARATE.get(src, []) + [
            "-c", os.path.join(CSRC, src), "-o", obj]
        jobs.append((cmd, obj, src))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "4"))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda j: _run(j[0], verbose, f"compiling {j[2]}"), jobs))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + [j[1] for j in jobs] + ["-o", tmp],
         verbose, "linking libdg.so")
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    os.replace(tmp, LIB)
    return LIB


def resource_usage() -> str:
    """Per-kernel VGPR/SGPR/spill/LDS report of the device code (compile only)."""
    srcs = [s for s in SOURCES if s.endswith(".hip")]
    out = []
    for s in srcs:
        cmd = [HIPCC] + [f for f in FLAGS if f not in ("-shared",)] + SEPARATE.get(s, []) + [
            "--cuda-device-only", "-c", "-Rpass-analysis=kernel-resource-usage",
            os.path.join(CSRC, s), "-o", os.devnull]
        res = subprocess.run(cmd, capture_output=True, text=True)
        out.append(res.stderr)
    return "\n".join(out)


if __name__ == "__main__":
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        sys.exit(f"hipcc not found at {HIPCC}")
    print(build(verbose=True))
    if "--usage" in sys.argv:
        print(resource_usage())
