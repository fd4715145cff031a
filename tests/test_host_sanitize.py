"""The C ABI's host-side validation (csrc/api.cpp) built with the host address and undefined-behaviour sanitizers
(g++, no device code: the kernel launchers are stubbed by tests/sanitize/launch_stubs.cpp) and driven through every
entry point's error paths and valid calls by tests/sanitize/abi_validation.cpp.  Runs on the CPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "token_eviction_scoring_amd", "csrc", "api.cpp"),
       os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
       os.path.join(ROOT, "tests", "sanitize", "abi_validation.cpp")]


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_abi_validation_under_host_sanitizers(tmp_path):
    exe = tmp_path / "abi_validation"
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "token_eviction_scoring_amd", "csrc"),
           *SRC, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # verify_asan_link_order=0: the environment may preload a library ahead of the sanitizer runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ok: 0 failures" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_precondition_checks_on_the_host(tmp_path):
    # the check kernel's per-sequence code (csrc/tri_checks.h) compiled for the host and fed bad inputs
    exe = tmp_path / "checks_host"
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "token_eviction_scoring_amd", "csrc"),
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(ROOT, "tests", "sanitize", "checks_host.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env)
    assert r.returncode == 0 and "ok: 0 failures" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
