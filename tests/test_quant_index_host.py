"""Index arithmetic of the block quantiser, checked on the host: every
global and LDS address the kernel forms, for d = 64, 128, 256 with and
without the rotation and ragged sequence lengths, through the same
functions the kernel calls (io_aware_exact_05_amd/csrc/fa_quant_index.h).
Includes the rebuilt 64-bit base address of the staged pass, whose low word
must stay unsigned (a sign-extended low word once sent that pass's copies
to a wild address).  Built with g++ under the address and undefined-
behaviour sanitizers; no GPU code is built or run."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_exact_05_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_quantiser_addresses_in_bounds_and_bijective():
    with tempfile.TemporaryDirectory(prefix="fa_qidx_") as tmp:
        exe = os.path.join(tmp, "qidx")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", "-I", CSRC,
               os.path.join(ROOT, "tests", "host", "quant_index_check.cpp"), "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
        assert "0 failures" in r.stdout, r.stdout
