"""Build the gfx950 HIP library libfa.so in-tree with hipcc.

The library holds the fused attention forward and backward kernels and their C ABI (include/fa.h).
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("fa_fwd.hip", "fa_bwd.hip", "gdn_fwd.hip")]
LIB = os.path.join(PKG, "libfa.so")
ARCH = os.environ.get("FA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU ops stay off: the compiler's plain scalar float code is used instead
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the Gated DeltaNet state walk (one wave per SIMD, so
    # more than 256 registers allowed) otherwise keeps its state and chunk products in AGPRs and
    # copies them to VGPRs every chunk; the attention kernels compile to the same code either way
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I" + os.path.join(ROOT, "include"),
    "-I" + os.path.join(PKG, "csrc"),
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def build(verbose: bool = False) -> str:
    """Always recompiles; returns the library path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + SRCS + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    # a shared library links even with unresolved symbols: resolve them all now, loudly
    import ctypes

    ctypes.CDLL(tmp, mode=os.RTLD_NOW)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
