"""The C ABI from C: tests/c_abi_consumer.c is compiled with gcc as strict C99 against
include/q2_0.h, linked against libq2_0.so and run.  It checks only host-side behaviour
(version, status strings, argument checks and empty no-ops), so it needs no GPU."""

import os
import shutil
import subprocess

import pytest

from ternary_bit_quantized_amd import q2_0 as B

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_against_the_header_and_library(tmp_path):
    lib = B.LIB_PATH
    assert os.path.exists(lib), "libq2_0.so is not built"
    exe = str(tmp_path / "consumer")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "c_abi_consumer.c"), "-o", exe, lib, "-Wl,-rpath," + os.path.dirname(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
