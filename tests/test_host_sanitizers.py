"""The host library's planner, cache and C ABI under sanitizers (CPU only).

tests/cpp/metadata_stress.cpp drives the C ABI from 16 threads (cache hits,
releases, clears, thread-local error messages) with host-only metadata. It is
linked with the library's host sources and kernel-launcher stand-ins, built
with g++ and ThreadSanitizer, then with AddressSanitizer plus
UndefinedBehaviorSanitizer, and must run clean.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "packed_sequence_causal_amd", "csrc")
ROCM = "/opt/rocm"

pytestmark = pytest.mark.skipif(
    shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")),
    reason="needs g++ and the HIP runtime library")


@pytest.mark.parametrize("sanitizer", ["thread", "address,undefined"])
def test_metadata_cache_is_clean_under_sanitizer(sanitizer, tmp_path):
    exe = str(tmp_path / "stress")
    sources = [os.path.join(CSRC, "thd_plan.cpp"), os.path.join(CSRC, "thd_api.cpp"),
               os.path.join(ROOT, "tests", "cpp", "launch_stubs.cpp"),
               os.path.join(ROOT, "tests", "cpp", "metadata_stress.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=" + sanitizer,
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include")] + sources + [
           "-L" + os.path.join(ROCM, "lib"), "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-lamdhip64", "-lpthread", "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1", ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0 and "ok" in run.stdout, (run.stdout + run.stderr)[-4000:]
