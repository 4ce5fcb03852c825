"""The C ABI's host layer (csrc/api.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer: built with g++/gcc together with a C driver
(tests/sanitize/abi_errors.c) and stand-in launchers
(tests/sanitize/launch_stubs.cpp), then run. The driver takes every entry point
through its argument-validation paths (none reaches a device), the workspace
size queries, the error names and profiling record, and the chunk selector,
whose choices are compared here with the oracle's selector. Any sanitizer
report aborts the run."""
import os
import shutil
import subprocess

import pytest

from oracle.selection import select_chunks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def build(tmp):
    gcc, gxx = shutil.which("gcc"), shutil.which("g++")
    if not gcc or not gxx or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("gcc/g++ or the HIP headers are not available")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include")]
    objs = []
    for src, cc, std in ((os.path.join(ROOT, "sequence_chunked_exact_amd", "csrc", "api.cpp"), gxx, "-std=c++17"),
                         (os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"), gxx, "-std=c++17"),
                         (os.path.join(ROOT, "tests", "sanitize", "abi_errors.c"), gcc, "-std=c99")):
        obj = os.path.join(tmp, os.path.basename(src) + ".o")
        subprocess.run([cc, std, *SAN, "-D__HIP_PLATFORM_AMD__", "-Wall", *inc, "-c", src, "-o", obj],
                       check=True, capture_output=True, text=True)
        objs.append(obj)
    exe = os.path.join(tmp, "abi_errors")
    lib = os.path.join(ROCM, "lib")
    subprocess.run([gxx, *SAN, *objs, "-L", lib, f"-Wl,-rpath,{lib}", "-lamdhip64", "-o", exe],
                   check=True, capture_output=True, text=True)
    return exe


def test_abi_host_layer_clean_under_asan_and_ubsan(tmp_path):
    exe = build(str(tmp_path))
    # verify_asan_link_order=0: the environment may preload a library ahead of
    # the ASan runtime, which is harmless for this host-only program
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=1:detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, (run.stdout[-3000:], run.stderr[-3000:])
    lines = run.stdout.splitlines()
    assert lines[-1].startswith("ok "), lines[-5:]
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr[-3000:]
    n = 0
    for ln in lines:
        if ln.startswith("select "):
            head, got = ln[len("select "):].split(":")
            k, t, seed = (int(x) for x in head.split())
            assert [int(x) for x in got.split()] == select_chunks(k, t, seed), ln
            n += 1
    assert n > 100
