"""The C ABI from a plain C99 program: tests/c_consumer/fa_c_consumer.c (HIP runtime C API for
memory, fa.h for the forward, the fp64 oracle for the check) is compiled with gcc against
libfa.so and run as a child process on a few shapes, including the error paths it checks."""
import os
import shutil
import subprocess
import sys

import pytest

import gqa_attention_forward_amd as fa
from oracle import build as oracle_build

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def consumer(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    lib_oracle = oracle_build.ensure_built()
    exe = str(tmp_path_factory.mktemp("c_consumer") / "fa_c_consumer")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), os.path.join(ROOT, "tests", "c_consumer", "fa_c_consumer.c"), "-o", exe,
           "-L", os.path.dirname(fa.LIB_PATH), "-lfa", "-L", os.path.dirname(lib_oracle), "-loracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath," + os.path.dirname(fa.LIB_PATH), "-Wl,-rpath," + os.path.dirname(lib_oracle),
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    return exe


@pytest.mark.parametrize("shape", [(1, 4, 2, 200, 300, 128, 1), (2, 8, 8, 129, 77, 64, 0), (1, 8, 2, 1, 1000, 128, 1)])
def test_c_consumer(consumer, shape):
    r = subprocess.run([consumer] + [str(x) for x in shape], capture_output=True, text=True, timeout=120)
    sys.stdout.write(r.stdout)
    sys.stderr.write(r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
