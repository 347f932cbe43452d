"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers under tests/sanitize/ are compiled with gcc/g++ and
-fsanitize=address,undefined (every error fatal) and run:
  * oracle_driver.c with oracle/oracle.c: every oracle entry point on tiny
    inputs (fp64, fp32 and bf16 inputs, several threads, causal and not, more
    queries than keys, an empty decode sequence, invalid arguments), with the
    closed forms a single key and an empty sequence fix;
  * abi_driver.cpp with exact_io_aware_fa_amd/csrc/fa_api.cpp: the C ABI's
    argument validation and workspace carving for every entry point, with the
    kernel launchers replaced by stubs (no GPU is touched).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd_build, exe, marker, tmp_path):
    r = subprocess.run(cmd_build, capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, "build failed:\n" + r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and marker in r.stdout, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-pthread"] + SAN + ["tests/sanitize/oracle_driver.c", "oracle/oracle.c", "-lm",
                                                  "-o", exe], exe, "ORACLE SANITIZE OK", tmp_path)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers are missing")
def test_abi_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    _run(["g++", "-std=c++17"] + SAN + ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-Iinclude",
                                        "-Iexact_io_aware_fa_amd/csrc", "tests/sanitize/abi_driver.cpp",
                                        "exact_io_aware_fa_amd/csrc/fa_api.cpp", "-o", exe],
         exe, "ABI SANITIZE OK", tmp_path)
