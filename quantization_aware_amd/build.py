"""Build libquest.so in-tree with hipcc for gfx950.

Each translation unit is compiled by its own hipcc process (in parallel),
then the objects are linked into the shared library.

Usage: python -m quantization_aware_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libquest.so")
SOURCES = [
    "quest_api.hip",
    "quest_launch.hip",
    "quest_fwd_nodq.hip",
    "quest_fwd_dq_bf16.hip",
    "quest_fwd_dq_f32.hip",
    "quest_fwd_op.hip",
    "quest_gemm.hip",
    "quest_grids.hip",
]
# Sources built without the VGPR-only MFMA form, leaving the placement of the
# matrix-core accumulators to the register allocator (the product kernel, whose
# 128 accumulator registers per wave share the 256-register budget of two
# waves per SIMD: the VGPR-only form spilled there).
AGPR_SOURCES = {"quest_gemm.hip"}
ARCH = "gfx950"
NOISE = "is not a recognized feature for this target"  # the host pass does not know the GPU feature below


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libquest needs ROCm's hipcc to build")


def compile_flags(source: str = "") -> list[str]:
    vgpr_form = [] if source in AGPR_SOURCES else ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        # Packed fp32 VALU forms are kept out of every kernel.
        "-Xclang",
        "-target-feature",
        "-Xclang",
        "-packed-fp32-ops",
        # Matrix-core results go straight to VGPRs (no accumulator-register
        # copies), except in the sources listed in AGPR_SOURCES.
        *vgpr_form,
        "-I",
        os.path.join(ROOT, "include"),
    ]


def compile_command(source: str, obj: str) -> list[str]:
    return [hipcc_path(), *compile_flags(source), "-c", os.path.join(CSRC, source), "-o", obj]


def link_command(objs: list[str], out_path: str) -> list[str]:
    return [hipcc_path(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_path, *objs]


def _run(cmd: list[str], verbose: bool) -> None:
    res = subprocess.run(cmd, capture_output=True, text=True)
    text = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if NOISE not in line)
    if res.returncode != 0:
        sys.stderr.write(text + "\n")
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd)}")
    if verbose and text.strip():
        print(text)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile libquest.so next to this file (every time) and return its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        list(pool.map(lambda so: _run(compile_command(*so), verbose), zip(SOURCES, objs)))
    tmp = LIB_PATH + ".tmp"
    _run(link_command(objs, tmp), verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
