"""The host-side ABI tests (test_abi.py) once more, against a build of the library whose
host code carries AddressSanitizer and UndefinedBehaviorSanitizer checks: argument
validation, the status strings and the export table run without a memory error or
undefined behaviour.  CPU only (no call launches a kernel); the build takes ~20 s."""

import os
import subprocess
import sys

from ternary_bit_quantized_amd import build as BUILD

HERE = os.path.dirname(os.path.abspath(__file__))


def test_abi_under_asan_and_ubsan():
    lib = BUILD.build_sanitized()
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in out and "__ubsan_handle" in out, "the build is not instrumented"
    env = BUILD.sanitized_env()
    which = subprocess.run([sys.executable, "-c", "from ternary_bit_quantized_amd import q2_0 as B; print(B.LIB_PATH)"],
                           env=env, capture_output=True, text=True, timeout=120)
    assert which.stdout.strip() == lib, which.stdout + which.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi.py")],
                       env=env, capture_output=True, text=True, timeout=600)
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-4000:]
    assert "ERROR: AddressSanitizer" not in text and "runtime error:" not in text, text[-4000:]
    assert " passed" in text
