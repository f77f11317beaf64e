"""The host library (fp_api.cpp: validation, plan bookkeeping, memory cache, stream and
event handling, every error path) built for the host alone with address and
undefined-behaviour sanitizers, against a stub HIP runtime in which any one
runtime call can be made to fail (tests/host/hip_stub.cpp), and driven by
tests/host/host_driver.cpp: every API scenario succeeds as is and fails
cleanly -- FP_ERR_OOM or FP_ERR_HIP, a message, no plan handed out, no
memory, event or stream left -- with each of its fallible calls failing in
turn.  No GPU is needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_long_context_last_amd", "csrc")
INC = os.path.join(ROOT, "include")
HOST = os.path.join(ROOT, "tests", "host")
ROCM = "/opt/rocm"

pytestmark = pytest.mark.slow


def _tools():
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not found")
    return hipcc, clang


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{out}"
    return out


def test_host_library_error_paths_under_sanitizers(tmp_path):
    hipcc, clang = _tools()
    common = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-I", CSRC, "-I", INC]
    # host-only HIP compilation; each sanitizer flag applies to the host pass
    san_host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined"]
    for src, obj in ((os.path.join(CSRC, "fp_api.cpp"), "fp_api.o"), (os.path.join(HOST, "hip_stub.cpp"), "stub.o")):
        _run([hipcc, "-x", "hip", "--offload-host-only", *common, *san_host, "-c", src, "-o", obj], tmp_path)
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    _run([clang, *common, *san, "-c", os.path.join(HOST, "host_driver.cpp"), "-o", "driver.o"], tmp_path)
    _run([clang, *san, "fp_api.o", "stub.o", "driver.o", "-o", "driver"], tmp_path)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(tmp_path / "driver")], cwd=tmp_path, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=300)
    print(r.stdout[-4000:])
    assert r.returncode == 0, r.stdout[-8000:]
    assert "check(s) failed" in r.stdout and " 0 check(s) failed" in r.stdout


def test_host_library_threads_under_thread_sanitizer(tmp_path):
    """Six threads plan, attend, read back and destroy plans at once while a
    seventh trims the memory cache and toggles the measurement hooks; the
    thread sanitizer must report no data race and every call must succeed."""
    hipcc, clang = _tools()
    common = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-I", CSRC, "-I", INC]
    tsan_host = ["-Xarch_host", "-fsanitize=thread"]
    for src, obj in ((os.path.join(CSRC, "fp_api.cpp"), "fp_api.o"), (os.path.join(HOST, "hip_stub.cpp"), "stub.o")):
        _run([hipcc, "-x", "hip", "--offload-host-only", *common, *tsan_host, "-c", src, "-o", obj], tmp_path)
    tsan = ["-fsanitize=thread"]
    _run([clang, *common, *tsan, "-c", os.path.join(HOST, "threads_driver.cpp"), "-o", "driver.o"], tmp_path)
    _run([clang, *tsan, "fp_api.o", "stub.o", "driver.o", "-lpthread", "-o", "driver"], tmp_path)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 second_deadlock_stack=1")
    r = subprocess.run([str(tmp_path / "driver")], cwd=tmp_path, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=300)
    print(r.stdout[-4000:])
    assert r.returncode == 0, r.stdout[-8000:]
    assert "ThreadSanitizer" not in r.stdout
    assert " 0 failure(s)" in r.stdout
