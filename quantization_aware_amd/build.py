"""Build libquest.so in-tree with hipcc for gfx950.

Usage: python -m quantization_aware_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libquest.so")
SOURCES = ["quest_api.hip", "quest_kernels.hip"]
ARCH = "gfx950"


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libquest needs ROCm's hipcc to build")


def build_command(out_path: str = LIB_PATH) -> list[str]:
    return [
        hipcc_path(),
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        # Packed fp32 VALU forms are kept out of every kernel.
        "-Xclang",
        "-target-feature",
        "-Xclang",
        "-packed-fp32-ops",
        # Matrix-core results go straight to VGPRs (no accumulator-register copies).
        "-mllvm",
        "-amdgpu-mfma-vgpr-form",
        "-I",
        os.path.join(ROOT, "include"),
        "-o",
        out_path,
        *[os.path.join(CSRC, s) for s in SOURCES],
    ]


def build(verbose: bool = False) -> str:
    """Compile libquest.so next to this file and return its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = build_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose:
        noise = "is not a recognized feature for this target"
        for line in (res.stdout + res.stderr).splitlines():
            if noise not in line:
                print(line)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
