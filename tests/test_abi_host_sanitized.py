"""Argument validation and dispatch of the C ABI layer (api.cpp), built for
the host alone with the address and undefined-behaviour sanitizers: every
status of a table of valid and invalid calls (null pointers, shapes at and
past the indexing limits, dtypes, head dimensions, alignment, aliasing,
workspace sizes) and the key/value-cache cut (whole chunks covering the
cache, workspace size) without a device.  The kernel launchers are stubs in
tests/host/abi_host_driver.cpp, so no GPU code is built or run."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_exact_05_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_abi_validation_under_sanitizers():
    with tempfile.TemporaryDirectory(prefix="fa_abi_host_") as tmp:
        exe = os.path.join(tmp, "abi_host")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
               "-I", CSRC, os.path.join(CSRC, "api.cpp"),
               os.path.join(ROOT, "tests", "host", "abi_host_driver.cpp"), "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
        assert "0 failures" in r.stdout, r.stdout
