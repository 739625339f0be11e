"""The host partitioner under AddressSanitizer and UBSan, and under
ThreadSanitizer on four threads: tests/c/partition_fuzz.cpp
with plan.cpp and api.cpp, built for the host by g++ (the GPU launchers are
stubbed in the driver), runs 1200 random decode, prefill and cascade
partitions, with output arrays sized exactly to the reported counts and one
entry short, and checks their invariants.  Any sanitizer report fails the
test.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_gqa_decode_pa_amd", "csrc")


def _build(tmp_path, sanitizers):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    exe = tmp_path / "partition_fuzz"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *sanitizers,
           "-D__HIP_PLATFORM_AMD__", "-isystem", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "c", "partition_fuzz.cpp"),
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "api.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-lpthread", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return exe


def test_partitioner_under_sanitizers(tmp_path):
    exe = _build(tmp_path, ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"])
    env = {**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0", "UBSAN_OPTIONS": "print_stacktrace=1"}
    r = subprocess.run([str(exe), "1200"], capture_output=True, text=True, timeout=600, env=env)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-3000:]
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-3000:]
    assert "0 failures" in r.stdout


def test_partitioner_threads_under_tsan(tmp_path):
    """Partitions computed on four host threads at once (no shared state
    but the thread-local error detail): ThreadSanitizer reports nothing."""
    exe = _build(tmp_path, ["-fsanitize=thread"])
    r = subprocess.run([str(exe), "150", "4"], capture_output=True, text=True, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-3000:]
    assert "ThreadSanitizer" not in report, report[-3000:]
    assert "0 failures" in r.stdout
