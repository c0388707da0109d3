"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds, each loaded into a fresh Python process with the sanitizer
runtime preloaded and every report fatal:
  * the oracle (plain C, gcc) with address, undefined and float-cast-overflow
    checks, running every oracle pin: a cast of a NaN or an out-of-range value
    to an integer type, a signed overflow or an out-of-bounds access in the
    oracle aborts the run;
  * the HIP library with its host code (argument checks, sizes, dispatch)
    instrumented (device code is unchanged), running the C-ABI boundary tests,
    which reach every rejection path without a GPU.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "qgemm_oracle.c")
ORACLE_PINS = [os.path.join(ROOT, "tests", f) for f in (
    "test_oracle_int4.py", "test_oracle_int8.py", "test_oracle_w4a8_g32.py",
    "test_oracle_int4_dq.py", "test_oracle_intn.py")]
SAN_OPTS = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
            "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run_pytest(files, env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-pthread", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "oracle"), ORACLE_SRC, "-o", lib, "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    env = dict(os.environ, QGEMM_ORACLE_LIB=lib, LD_PRELOAD=asan, **SAN_OPTS)
    _run_pytest(ORACLE_PINS, env)


def test_boundary_under_asan_and_ubsan_host_code(tmp_path):
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    sys.path.insert(0, os.path.join(ROOT, "gemm_decode_qgemm_amd"))
    try:
        import build as hip_build
    finally:
        sys.path.pop(0)
    host_san = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-shared-libasan",
                "-Xarch_host", "-fno-omit-frame-pointer"]
    clangxx = "/opt/rocm/llvm/bin/clang++"
    link = [clangxx, "-fsanitize=address,undefined", "-shared-libasan",
            "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    lib = str(tmp_path / "libqgemm_san.so")
    hip_build.build(out=lib, extra=host_san, objdir=str(tmp_path / "obj"), link=link)
    env = dict(os.environ, QGEMM_LIB=lib, LD_PRELOAD=rt[-1], **SAN_OPTS)
    _run_pytest([os.path.join(ROOT, "tests", "test_boundary.py")], env)
