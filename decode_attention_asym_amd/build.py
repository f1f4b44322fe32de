"""Build libkvq.so (all HIP kernels + the C-ABI host code) for gfx950, in-tree."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["kvq_api.cpp", "kvq_plan.cpp", "kvq_quant.hip", "kvq_decode_generic.hip",
           "kvq_decode_gqa.hip", "kvq_decode_mha.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms stay off (only scalar / non-packed fp32 code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # MFMA accumulators in VGPRs (no AGPR copies around VALU work on them)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def build(verbose: bool = False) -> str:
    """Compile every source into libkvq.so (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True, cwd=CSRC)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
