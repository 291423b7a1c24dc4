"""Build libfp8blk.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfp8blk.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: every fused multiply-add in the kernels is written out
# explicitly, nothing else may be contracted. "-Xclang -target-feature -Xclang
# -packed-fp32-ops" turns packed FP32 instructions off in the gfx950 device
# pass; the host (x86) pass does not know the feature and prints "not a
# recognized feature for this target", which is harmless.
# tests/test_build_code.py disassembles the built code objects and checks
# that no packed FP32 add, multiply or fused multiply-add is left (and that no
# kernel spills to scratch). f32 subnormals are kept (the default; stated for
# the reader).
# Matrix-core accumulators live in ordinary VGPRs (-amdgpu-mfma-vgpr-form):
# with AGPR accumulators the compiler copies them between the two register
# files around every loop iteration of the sequence kernel.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-Wall", "-Wno-unused-command-line-argument",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# hipBLASLt provides the staged prefill path's bf16 GEMM.
LIBS = ["-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"]


def command(out: str = LIB) -> list[str]:
    return [HIPCC, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", out, *sources(), *LIBS]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into the shared library next to this file."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
