"""The C ABI consumed from plain C: tests/c_abi_check.c includes
include/packed_bit_gemv.h, is compiled by gcc as C99 and linked against the
built library, and checks the helpers and the argument checks of every entry
point (all calls invalid on purpose, so no GPU is needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "packed_bit_gemv_amd")
LIB = os.path.join(PKG, "libpackedbitgemv.so")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_consumer(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("library not built")
    exe = tmp_path / "c_abi_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{ROCM_INCLUDE}", os.path.join(ROOT, "tests", "c_abi_check.c"),
           f"-L{PKG}", "-lpackedbitgemv", f"-Wl,-rpath,{PKG}", "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
