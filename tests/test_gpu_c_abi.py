"""The C ABI used from a plain C program on the GPU: no Python, no torch, only
include/ar.h, libar.so and the HIP runtime (tests/c_abi/abi_gpu_check.c)."""

import os
import shutil
import subprocess

import pytest

from gpu_util import require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_plain_c_program_on_the_gpu(tmp_path):
    require_gpu()
    from ring_allreduce_reduction_virtual_amd import _lib

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    libdir = os.path.dirname(_lib.LIB_PATH)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = tmp_path / "abi_gpu_check"
    print("[c abi] building the C program", flush=True)
    subprocess.run([gcc, "-std=c99", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
                    os.path.join(ROOT, "tests", "c_abi", "abi_gpu_check.c"),
                    "-L", libdir, "-l:libar.so", f"-Wl,-rpath,{libdir}",
                    "-L", os.path.join(rocm, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}",
                    "-o", str(exe)], check=True, capture_output=True, text=True)
    print("[c abi] running it", flush=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=100)
    print(res.stdout)
    assert res.returncode == 0, res.stderr
    assert "ar.h GPU checks passed" in res.stdout
