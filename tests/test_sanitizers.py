"""CPU runs of the oracle and of the C-ABI's host-side validation under
AddressSanitizer and UndefinedBehaviorSanitizer (gcc / g++ builds of the
plain C and C++ sources; the GPU kernels are not part of these builds: the
C-ABI layer is linked against host stand-ins of its kernel launchers and of
the two HIP device queries, tests/sanitize/api_stubs.cpp)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1"]
HIP_INC = "/opt/rocm/include"


def _build(cmd, tmp_path):
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp_path)
    if r.returncode != 0:
        if "asan" in r.stderr.lower() or "sanitizer" in r.stderr.lower():
            pytest.skip("no sanitizer runtime for this compiler")
        raise AssertionError(r.stdout + r.stderr)


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_drv")
    _build(["gcc", "-std=c11", "-ffp-contract=off", *SAN, os.path.join(ROOT, "oracle", "oracle.c"),
            os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-o", exe, "-lm"], tmp_path)
    assert "oracle checks ok" in _run(exe)


@pytest.mark.skipif(not os.path.isdir(HIP_INC), reason="HIP headers not installed")
def test_abi_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "api_drv")
    src = os.path.join(ROOT, "gguf_quantized_matvec_amd", "csrc", "qmv_api.cpp")
    _build(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INC, *SAN, src,
            os.path.join(ROOT, "tests", "sanitize", "api_stubs.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp"), "-o", exe], tmp_path)
    assert "api checks ok" in _run(exe)
