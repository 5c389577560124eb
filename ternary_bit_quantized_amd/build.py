"""Build libq2_0.so (HIP for gfx950) in-tree with hipcc.

Usage: python -m ternary_bit_quantized_amd.build [--sanitize]
Every source in csrc/ is compiled for gfx950 only; object files go to _build/ at the
repository root and the shared library next to this file.  The measurement kernels in
ceilings/ (HBM read stream, MFMA loop, empty launch, and a probe of the matrix cores'
rounding) become libq2_0_ceilings.so, which only the benchmark and the tests load.

--sanitize builds a second copy, _build/sanitize/libq2_0.so, whose host code carries
AddressSanitizer and UndefinedBehaviorSanitizer checks (device code as usual).  It is for
the host-side ABI tests: load it with Q2_0_LIB=<path> and the clang ASan runtime
preloaded (sanitized_env() gives that environment).
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libq2_0.so")
CEIL_SRC = os.path.join(PKG, "ceilings", "ceilings.hip")
CEIL_LIB = os.path.join(PKG, "libq2_0_ceilings.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMPILE_TIMEOUT_S = 600
# Packed-FP32 VALU forms are switched off for all device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


# MFMA results straight into VGPRs (no v_accvgpr_read per result) where the
# kernel consumes them with VALU ops right away.
PER_FILE = {"mat_vec_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
            "mat_vec_stream.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *PER_FILE.get(os.path.basename(src), []), "-c", src, "-o", obj]
    # a compile that runs away (the scheduler on some inputs) fails instead of hanging
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=COMPILE_TIMEOUT_S)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=COMPILE_TIMEOUT_S)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        objs = list(ex.map(_compile, srcs + [CEIL_SRC]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], CEIL_LIB)
    if verbose:
        print("built", LIB, "and", CEIL_LIB)
    return LIB


SAN_DIR = os.path.join(BUILD, "sanitize")
# host code only: each sanitizer flag applies to the host pass alone
SAN_FLAGS = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def asan_runtime() -> str:
    """The ASan runtime of hipcc's clang (it carries the UBSan handlers too)."""
    llvm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    hits = sorted(glob.glob(os.path.join(llvm, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")) +
                  glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so next to " + HIPCC)
    return hits[-1]


def sanitized_env(base=None) -> dict:
    """Environment for a process that loads the sanitized library: the library path, the
    ASan runtime ahead of any preload already set, leaks off (the interpreter is not
    instrumented), every report fatal."""
    env = dict(os.environ if base is None else base)
    env["Q2_0_LIB"] = os.path.join(SAN_DIR, "libq2_0.so")
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = asan_runtime() + (":" + pre if pre else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def build_sanitized(verbose: bool = False) -> str:
    os.makedirs(SAN_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def comp(src):
        obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, *SAN_FLAGS, *PER_FILE.get(os.path.basename(src), []), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=COMPILE_TIMEOUT_S)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(comp, srcs))
    lib = os.path.join(SAN_DIR, "libq2_0.so")
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp, "-shared-libasan", *SAN_FLAGS[1:]]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=COMPILE_TIMEOUT_S)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
