"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs are built with g++ and run:
  * the C ABI's validation and dispatch (api.cpp) linked with stand-in
    launchers (tests/host_sanitize/launch_stubs.cpp), driven through valid and
    invalid arguments of every entry point (tests/host_sanitize/api_driver.cpp);
  * the CPU oracle (oracle/oracle.cpp) on small inputs and edge cases
    (tests/host_sanitize/oracle_driver.cpp).
Any memory error, undefined behaviour or leak ends the program with a nonzero
status.  No GPU code is built or run.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
SAN = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
       "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


def build_and_run(tmp_path, name, sources, extra):
    exe = str(tmp_path / name)
    r = subprocess.run(["g++"] + SAN + extra + sources + ["-o", exe], capture_output=True,
                       text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("the sanitizer runtimes are not installed")
    assert r.returncode == 0, r.stderr
    return subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)


def test_api_validation_under_sanitizers(tmp_path):
    r = build_and_run(
        tmp_path, "api_san",
        [os.path.join(ROOT, "kv_cache_eviction_05_amd", "csrc", "api.cpp"),
         os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "api_driver.cpp")],
        ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
         "-I", os.path.join(ROOT, "kv_cache_eviction_05_amd", "csrc")])
    assert r.returncode == 0, r.stdout + r.stderr
    assert "api ok" in r.stdout


def test_oracle_under_sanitizers(tmp_path):
    r = build_and_run(tmp_path, "oracle_san",
                      [os.path.join(ROOT, "oracle", "oracle.cpp"),
                       os.path.join(HERE, "oracle_driver.cpp")], [])
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle ok" in r.stdout
