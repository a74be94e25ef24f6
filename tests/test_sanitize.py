"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer runs (CPU only).

* The CPU oracle (oracle/moe_oracle.c) with tests/sanitize/oracle_driver.c: every
  oracle entry point on small layers, with empty experts, k = E, one and zero tokens,
  and invalid routing.
* The library's host code (csrc/moe_api.cpp) with tests/sanitize/host_driver.cpp and
  failing stubs in place of the kernel launchers: plan validation, workspace layout,
  the memory report into buffers of every length, status strings and host refusals.

Both are built with gcc / g++ (-fsanitize=address,undefined, no recovery) and must
exit 0 with no sanitizer report.  GPU code is never built with a sanitizer here.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(exe):
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "runtime error" not in r.stdout and "AddressSanitizer" not in r.stdout, r.stdout[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.check_call(["gcc", "-std=c11", "-fopenmp"] + SAN +
                          [os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                           os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm", "-o", exe])
    assert "ok" in _run(exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/lib/libamdhip64.so"),
                    reason="g++ or the HIP runtime library not installed")
def test_host_library_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_driver")
    subprocess.check_call(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-w"] + SAN +
                          [os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
                           os.path.join(ROOT, "mixture_experts_routed_dispatch_amd", "csrc", "moe_api.cpp"),
                           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    assert "ok" in _run(exe)
