"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

api.cpp (argument validation, launch planning, workspace layout, planner introspection) and the
scheduler functions of plan.hpp it calls are compiled by the host compiler with
-fsanitize=address,undefined and linked with host-only launch stubs (tests/host/launch_stubs.cpp)
into a separate library.  A child Python process loads it in place of the GPU library (the
binding's ATTNFWD_LIB), with the ASan runtime preloaded, and runs every test of
tests/test_boundary.py plus the valid-argument calls of tests/host/sanitized_calls.py; any
sanitizer report fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_attn_fwd_03_amd", "csrc")


def _runtime(cxx, name):
    out = subprocess.run([cxx, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_c_abi_host_code_under_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    asan = _runtime(cxx, "libasan.so")
    if asan is None:
        pytest.skip("no AddressSanitizer runtime")
    lib = str(tmp_path / "libattnfwd_hostsan.so")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "api.cpp"), os.path.join(ROOT, "tests", "host", "launch_stubs.cpp"), "-o", lib]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ATTNFWD_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", CUDA_VISIBLE_DEVICES="", HIP_VISIBLE_DEVICES="")
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join(ROOT, "tests", "test_boundary.py"),
                          os.path.join(ROOT, "tests", "host", "sanitized_calls.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = run.stdout + run.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert run.returncode == 0, out[-4000:]
    assert " passed" in out and "skipped" not in out.split("\n")[-2], out[-1000:]
