"""The host layer (api.cpp: argument checks, stride / offset / overflow
arithmetic on caller sizes, the planner, workspace carving) built with g++
under AddressSanitizer and UndefinedBehaviorSanitizer, with the HIP runtime
and the kernel launchers replaced by host-only stubs
(tests/host_sanitize/), and the whole host ABI test file run against that
build.  Any sanitizer report, or a launcher stub's parameter check, fails
the run.  CPU only: no device is touched."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CSRC = os.path.join(ROOT, "sparse_mla_decode_gather_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")


def test_host_abi_tests_pass_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    so = str(tmp_path / "libsparsemla_sanitized.so")
    build = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-shared", "-fPIC", "-Wall",
             f"-I{os.path.join(HERE, 'stub')}", f"-I{INCLUDE}", f"-I{CSRC}",
             os.path.join(CSRC, "api.cpp"), os.path.join(HERE, "stub_hip.cpp"),
             "-o", so]
    r = subprocess.run(build, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    libasan = subprocess.check_output([gxx, "-print-file-name=libasan.so"],
                                      text=True).strip()
    env = dict(os.environ)
    env["SPARSEMLA_LIB"] = so
    # the sanitizer runtime must come first among the preloaded libraries;
    # anything already preloaded stays, after it
    env["LD_PRELOAD"] = libasan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    which = subprocess.run(
        [sys.executable, "-c",
         "from sparse_mla_decode_gather_amd import lib; print(lib.load()._name)"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert which.returncode == 0, which.stdout + which.stderr
    assert which.stdout.strip().splitlines()[-1] == so
    run = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
         os.path.join("tests", "test_abi_host.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    for marker in ("AddressSanitizer", "runtime error:", "stub launch:"):
        assert marker not in out, out[-4000:]
    assert " passed" in run.stdout
