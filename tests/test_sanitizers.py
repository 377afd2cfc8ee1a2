"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- tests/sanitize/oracle_check.cpp runs every export of the oracle's C++ on ragged shapes.
- tests/sanitize/capi_check.cpp runs the C ABI's validation, layout and size-query code
  (csrc/capi.hip compiled for the host) with stub launchers, over valid and invalid calls.

Both are built with g++ (-fsanitize=address,undefined, no recovery) into a temporary
directory; a sanitizer report or a failed expectation fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1"]
ROCM_INCLUDE = "/opt/rocm/include"


def _build(cmd, tmp):
    r = subprocess.run(cmd, cwd=tmp, capture_output=True, text=True)
    if r.returncode != 0:
        if "asan" in r.stderr.lower() and "cannot find" in r.stderr.lower():
            pytest.skip("the sanitizer runtimes are not installed")
        raise AssertionError("build failed:\n" + r.stderr[-4000:])


def _run(exe, tmp):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], cwd=tmp, capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-6000:]
    return r.stdout


@pytest.fixture(scope="module")
def gxx():
    g = shutil.which("g++")
    if g is None:
        pytest.skip("g++ is not installed")
    return g


def test_oracle_under_sanitizers(gxx, tmp_path):
    exe = str(tmp_path / "oracle_check")
    _build([gxx, "-std=c++17", "-pthread", *SAN, os.path.join(ROOT, "tests", "sanitize", "oracle_check.cpp"),
            "-o", exe], str(tmp_path))
    assert "oracle checks: ok" in _run(exe, str(tmp_path))


def test_c_abi_host_code_under_sanitizers(gxx, tmp_path):
    if not os.path.isdir(os.path.join(ROCM_INCLUDE, "hip")):
        pytest.skip("the HIP headers are not installed")
    exe = str(tmp_path / "capi_check")
    obj = str(tmp_path / "capi.o")
    hip = ["-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INCLUDE]
    _build([gxx, "-std=c++17", "-x", "c++", *hip, *SAN, "-c",
            os.path.join(ROOT, "bit_quantized_attention_03_amd", "csrc", "capi.hip"), "-o", obj], str(tmp_path))
    _build([gxx, "-std=c++17", *hip, *SAN, os.path.join(ROOT, "tests", "sanitize", "capi_check.cpp"), obj,
            "-o", exe], str(tmp_path))
    assert "capi host checks: ok" in _run(exe, str(tmp_path))
