"""The library's host code — argument validation, work planning, the CA-task
scheduler and the ring planning — built with AddressSanitizer and
UndefinedBehaviorSanitizer by the host compiler (no device code; kernel
launchers are stubs) and driven with random, mostly invalid, arguments.  Any
sanitizer report fails the test.  CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_core_amd", "csrc")
FUZZ = os.path.join(ROOT, "tests", "host_fuzz")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-D__bf16=unsigned short",
         "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def build_and_run(tmp_path, name, sources, libs=()):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")):
        pytest.skip("g++ or the HIP headers are not available")
    exe = str(tmp_path / name)
    cmd = [gxx] + FLAGS + sources + list(libs) + ["-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-3000:]
    return out


def test_scheduler_and_ring_planning_under_sanitizers(tmp_path):
    out = build_and_run(tmp_path, "sched_ring_fuzz",
                        [os.path.join(FUZZ, "sched_ring_fuzz.cpp"), os.path.join(CSRC, "ca_sched.cpp"),
                         os.path.join(CSRC, "ca_ring.cpp")])
    assert "host fuzz done" in out


def test_validation_and_planning_under_sanitizers(tmp_path):
    lib = os.path.join(ROCM, "lib")
    if not os.path.exists(os.path.join(lib, "libamdhip64.so")):
        pytest.skip("libamdhip64 is not available")
    out = build_and_run(tmp_path, "api_fuzz", [os.path.join(FUZZ, "api_fuzz.cpp"), os.path.join(CSRC, "ca_api.cpp")],
                        ["-L" + lib, "-lamdhip64", "-Wl,-rpath," + lib])
    assert "api host fuzz done" in out
