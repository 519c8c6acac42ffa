"""The C ABI used from plain C: tests/c/abi_check.c is compiled by gcc
against include/mn_norm.h (no HIP headers), linked against libmn_norm.so and
run; it exercises only host-side validation, so it needs no GPU."""
import os
import shutil
import subprocess

import pytest

import row_wise_normalization_amd as mn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not os.path.exists(mn.LIB_PATH), reason="libmn_norm.so not built")
@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_plain_c_caller(tmp_path):
    exe = os.path.join(tmp_path, "abi_check")
    libdir = os.path.dirname(mn.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I",
                    os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_check.c"),
                    "-L", libdir, "-lmn_norm", f"-Wl,-rpath,{libdir}", "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "ok"
