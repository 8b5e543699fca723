"""The host code of the C ABI (argument validation, error text, dispatch)
under AddressSanitizer and UndefinedBehaviorSanitizer: api.cpp is built with
g++ as a host-only library whose kernel launchers are stubs that report no
device (tests/sanitize/host_stubs.cpp), and tests/test_abi.py runs against it
in a subprocess with the sanitizer runtime preloaded.  Any report fails the
run (halt_on_error).  Needs g++ with libasan and the ROCm headers; skipped
otherwise.  No GPU code is built or run."""

import os
import shutil
import subprocess
import sys
import tempfile

import pytest

from tests.util import ROOT

ROCM = "/opt/rocm"


def _runtime(name):
    out = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_c_abi_validation_under_asan_and_ubsan():
    if shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")):
        pytest.skip("needs g++ and the ROCm headers")
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("libasan not found")
    tmp = tempfile.mkdtemp(prefix="mxq_asan_")
    try:
        lib = os.path.join(tmp, "libmxq_host_asan.so")
        csrc = os.path.join(ROOT, "microscaling_quantization_block_amd", "csrc")
        build = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined",
                 "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
                 "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", csrc,
                 os.path.join(csrc, "api.cpp"), os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"),
                 "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
                 "-o", lib]
        r = subprocess.run(build, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ)
        env.update(LD_PRELOAD=asan, MXQ_TEST_SANITIZED_LIBRARY=lib,
                   ASAN_OPTIONS="detect_leaks=0:detect_odr_violation=0:halt_on_error=1:abort_on_error=0",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_abi.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        report = r.stdout[-4000:] + r.stderr[-4000:]
        assert r.returncode == 0, report
        assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in report and "runtime error" not in report
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
