"""Build libspecverify.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libspecverify.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["sv_api.cpp", "sv_kernels.hip", "sv_measure.hip", "sv_noalloc.hip"]
ARCH = "gfx950"


def hipcc_command(out_path: str = LIB_PATH, extra=()) -> list[str]:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-fvisibility=hidden", "-I", INCLUDE, "-I", CSRC,
            # packed FP32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            *extra, *[os.path.join(CSRC, s) for s in SOURCES], "-o", out_path]


def build(out_path: str = LIB_PATH, extra=()) -> str:
    """Compile the library (always recompiles).  Writes to a temporary name
    first so a failed build never leaves a half-written library behind."""
    tmp = out_path + ".tmp"
    subprocess.run(hipcc_command(tmp, extra), check=True, cwd=CSRC)
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build())
