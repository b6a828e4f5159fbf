"""The C ABI from plain C, without Python or HIP headers: include/ulysses.h compiles as C11
with warnings as errors, a program links against libulysses.so, and the host-side argument
checks, status strings and workspace queries answer without a GPU (tests/c/abi_from_c.c)."""
import os
import shutil
import subprocess

import pytest

import ulysses_sequence_parallelism_rank_amd as U

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_from_plain_c(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    U.lib()  # raises when the library has not been built
    libdir = os.path.dirname(U.LIB_PATH)
    exe = str(tmp_path / "abi_from_c")
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-o", exe, "-L", libdir, "-lulysses",
           f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "c abi ok" in r.stdout, r.stdout + r.stderr
