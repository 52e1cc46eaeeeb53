"""The host C++ (schedule driver, argument checks) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

The driver and the checks are built with the recording fake backend
(tests/host/fake_backend.cpp) by g++ with -fsanitize=address,undefined (host
code only: no GPU code is involved).  Two programs run against that build:
  * a plain C99 client of the schedule API (tests/host/sched_c_client.c),
    built with the same sanitizers, leak checking on;
  * the host schedule tests (tests/test_schedule_host.py) in a Python
    process with the sanitizer runtime preloaded (leak checking off: the
    interpreter itself keeps memory until exit).
Any sanitizer report, or a non-zero exit, fails the test.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_bidirectional_attention_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
REPORTS = ("ERROR: AddressSanitizer", "ERROR: LeakSanitizer", "runtime error:")


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    if _runtime("libasan.so") is None or _runtime("libubsan.so") is None:
        pytest.skip("the gcc sanitizer runtimes are not installed")
    out = tmp_path_factory.mktemp("san")
    lib = str(out / "libsdattn_fake_san.so")
    srcs = [os.path.join(CSRC, "host_common.cpp"), os.path.join(CSRC, "schedule.cpp"),
            os.path.join(HOST, "fake_backend.cpp")]
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", *SAN, "-I", CSRC, "-I", os.path.join(ROOT, "include"),
                    *srcs, "-o", lib], check=True, capture_output=True, text=True)
    return out, lib


def _clean(text):
    for r in REPORTS:
        assert r not in text, text[-4000:]


def test_schedule_c_client_under_sanitizers(san_lib):
    out, lib = san_lib
    exe = str(out / "sched_c_client")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", *SAN, "-I", os.path.join(ROOT, "include"),
                    os.path.join(HOST, "sched_c_client.c"), "-o", exe, lib, f"-Wl,-rpath,{out}"],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    _clean(r.stdout + r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "schedule C client OK" in r.stdout
    assert "sparsed_64k: 205 dense, 0 dense+select, 1 select+sparse, 818 sparse" in r.stdout


def test_host_schedule_tests_under_sanitizers(san_lib):
    _, lib = san_lib
    preload = ":".join([_runtime("libasan.so"), _runtime("libubsan.so")])
    env = dict(os.environ, LD_PRELOAD=preload, SDATTN_FAKE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_schedule_host.py")],
                       capture_output=True, text=True, timeout=600, env=env, cwd=ROOT)
    _clean(r.stdout + r.stderr)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert " passed" in r.stdout
