"""Build libkvq.so (all HIP kernels + the C-ABI host code) for gfx950, in-tree."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms stay off (only scalar / non-packed fp32 code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
]
# MFMA accumulators in VGPRs (no AGPR copies around VALU work on them): for
# kernels whose accumulators fit next to everything else in 256 VGPRs
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]

# source -> extra flags
SOURCES = {
    "kvq_api.cpp": VGPR_FORM,
    "kvq_plan.cpp": VGPR_FORM,
    "kvq_quant.hip": VGPR_FORM,
    "kvq_decode_generic.hip": VGPR_FORM,
    "kvq_decode_gqa.hip": VGPR_FORM,
    "kvq_decode_mha.hip": VGPR_FORM,
    "kvq_decode_mla.hip": VGPR_FORM,
    "kvq_prefill.hip": VGPR_FORM,
    "kvq_noalloc.hip": [],
}
FLAGS = COMMON + VGPR_FORM   # kept for tools that print the main flag set


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *SOURCES[src], *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True, cwd=CSRC)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libkvq.so (always recompiles)."""
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True, cwd=CSRC)
    os.replace(tmp, LIB)
    return LIB


# ---- host-sanitizer build (CPU checks only): the C-ABI host code
# (argument checks, layout and split arithmetic) under AddressSanitizer and
# UndefinedBehaviorSanitizer, the kernels as in libkvq.so.  The sanitizers
# apply to the host pass only; load it with the clang ASan runtime preloaded
# (SAN_RUNTIME) and KVQ_LIB pointing at it.
SAN_LIB = os.path.join(HERE, "libkvq_san.so")
SAN_HOST = ["kvq_api.cpp", "kvq_plan.cpp"]
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
SAN_RUNTIME = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "lib", "llvm", "lib", "clang")


def san_runtime() -> str:
    """The clang ASan runtime that matches hipcc (to preload into Python)."""
    import glob
    hits = sorted(glob.glob(os.path.join(SAN_RUNTIME, "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("clang ASan runtime not found under " + SAN_RUNTIME)
    return hits[-1]


def build_sanitized(verbose: bool = False) -> str:
    """libkvq_san.so: SAN_HOST compiled with the host sanitizers, every other
    object taken from a fresh normal compile."""
    os.makedirs(OBJ, exist_ok=True)
    san_dir = os.path.join(OBJ, "san")
    os.makedirs(san_dir, exist_ok=True)

    def one(src):
        if src not in SAN_HOST:
            return _compile(src, verbose)
        obj = os.path.join(san_dir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *COMMON, *SOURCES[src], *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True, cwd=CSRC)
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = SAN_LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan", *SAN_FLAGS[:4], *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True, cwd=CSRC)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    print(build(verbose=True))
