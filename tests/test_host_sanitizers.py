"""The host part of the library -- slot pool, idle/pending state machine, argument validation,
prefill planning (kda_pool.cpp, kda_plan.cpp) -- built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, with tests/sanitize/hip_stubs.cpp standing in for the HIP runtime
and the kernel launchers, and the CPU ABI tests (tests/test_abi_cpu.py) run against that build
in a child process (KDA_LIB_PATH, the sanitizer runtime preloaded):

* ASan (leak checking off: the interpreter keeps its own allocations, and pointers to the
  pools, alive at exit) and UBSan, both stopping at the first error: the suite must pass;
* then tests/sanitize/host_abi_driver.cpp, a C++ program over the same host paths that
  destroys every pool it creates, under ASan with LeakSanitizer and UBSan: no error, no leak.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "recurrent_linear_attention_amd", "csrc")


SAN_FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
             "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
HOST_SOURCES = [os.path.join(CSRC, "kda_pool.cpp"), os.path.join(CSRC, "kda_plan.cpp"),
                os.path.join(ROOT, "tests", "sanitize", "hip_stubs.cpp")]


def _gxx():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan not available")
    return gxx, asan


def _compile(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]


def _run_abi_suite(lib, asan, asan_options):
    env = dict(os.environ, LD_PRELOAD=asan, KDA_LIB_PATH=lib, ASAN_OPTIONS=asan_options,
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return subprocess.run([sys.executable, "-m", "pytest", os.path.join("tests", "test_abi_cpu.py"),
                           "-x", "-q", "-p", "no:cacheprovider"],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def test_abi_cpu_suite_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    gxx, asan = _gxx()
    lib = str(tmp_path / "libkda_host_sanitized.so")
    _compile([gxx, "-shared", "-fPIC", *SAN_FLAGS, *HOST_SOURCES, "-Wl,--no-undefined", "-o", lib])
    r = _run_abi_suite(lib, asan, "detect_leaks=0:abort_on_error=1")
    out = r.stdout + r.stderr
    assert r.returncode == 0 and " passed" in r.stdout, out[-6000:]
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-6000:]


def test_host_driver_has_no_errors_and_no_leaks(tmp_path):
    gxx, _ = _gxx()
    exe = str(tmp_path / "host_abi_driver")
    _compile([gxx, *SAN_FLAGS, *HOST_SOURCES,
              os.path.join(ROOT, "tests", "sanitize", "host_abi_driver.cpp"), "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "host ABI driver: 0 failures" in r.stdout
    assert "Sanitizer" not in out and "runtime error" not in out, out[-6000:]
