"""The library's host C++ under AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp (planner, argument checks, error messages, the packing of launch
arguments) and kv_pool.cpp (the block allocator: all-or-nothing
allocation, refusal of freed handles, prefix sharing; lucebox PR #555, Summary
and Validation) are compiled with g++ -fsanitize=address,undefined into a
host-only build of the same C ABI, whose kernel launchers all refuse
(tests/host/launch_stubs.cpp). The library's CPU suites - the allocator's
model-based fuzz, the planner and refusal tests - and the calls that reach a
launcher (tests/host/sanitized_paths.py) then run against that build in a
child process with the sanitizer runtime preloaded; any report aborts the
child and fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_gqa_attn_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")
OUT_DIR = os.path.join(HOST, "_build")
LIB = os.path.join(OUT_DIR, "libpaged_attn_host_san.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _build():
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "kv_pool.cpp"),
            os.path.join(HOST, "launch_stubs.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", *srcs, f"-L{ROCM}/lib", "-lamdhip64", "-o", LIB + ".tmp"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stderr[-4000:]
    os.replace(LIB + ".tmp", LIB)


def test_host_code_under_address_and_undefined_behaviour_sanitizers():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("g++ has no AddressSanitizer runtime here")
    _build()
    env = dict(os.environ)
    env.update({
        "PAGED_ATTN_LIB": LIB,
        "LD_PRELOAD": asan,
        # Python and torch keep their allocations until exit by design
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "PYTHONPATH": os.pathsep.join([ROOT, os.path.join(ROOT, "tests")]),
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_kv_pool.py"), os.path.join(ROOT, "tests", "test_lib_cpu.py"),
           os.path.join(HOST, "sanitized_paths.py")]
    p = subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    tail = (p.stdout[-3000:] + "\n" + p.stderr[-6000:])
    assert p.returncode == 0, tail
    assert "AddressSanitizer" not in p.stderr and "runtime error" not in p.stderr, tail
    assert " passed" in p.stdout and "skipped" not in p.stdout.splitlines()[-1], tail
