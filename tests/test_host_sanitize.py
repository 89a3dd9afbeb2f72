"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

host.cpp (validation, planning, workspace carving, launch sequencing) and
plan.cpp (launch shapes) are compiled for the host alone with clang++ and
both sanitizers, with every kernel launcher replaced by a stub
(tests/sanitize/launch_stubs.cpp).  The ABI tests of test_host_abi.py then
run against that build, and tests/sanitize/orchestration_check.py drives
every entry point through a complete call for each workload (full,
windowed and int8 towers, merger, patch gather, fold, quantize).  Any
sanitizer report aborts the process and fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "resolution_vit_vision_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"


def _asan_runtime():
    if not os.path.exists(CLANG):
        return None
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang++ with the AddressSanitizer runtime is not available")
    out = str(tmp_path_factory.mktemp("san") / "libqv_stub_san.so")
    cmd = [CLANG, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-Wno-c++20-extensions",
           os.path.join(CSRC, "host.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1", QV_LIBRARY=out)
    return env


def _run(cmd, env):
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    text = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in text and "AddressSanitizer" not in text, text[-6000:]
    return text


def test_abi_tests_under_sanitizers(sanitized_lib):
    text = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                 os.path.join("tests", "test_host_abi.py")], sanitized_lib)
    assert " passed" in text


def test_full_orchestration_under_sanitizers(sanitized_lib):
    text = _run([sys.executable, os.path.join("tests", "sanitize", "orchestration_check.py")], sanitized_lib)
    assert "ran to completion" in text
