"""Compile the fp64 CPU oracles (attn_oracle.c, gdn_oracle.c) into oracle/liboracle.so with gcc.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use the library this builds.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, f) for f in ("attn_oracle.c", "gdn_oracle.c")]
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Always recompile; returns the path of the shared library."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math"] + SRCS + ["-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built() -> str:
    """Build when the library is missing or older than one of its sources."""
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < max(os.path.getmtime(f) for f in SRCS):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
