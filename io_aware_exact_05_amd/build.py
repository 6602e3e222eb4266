"""Build libfa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: ``python -m io_aware_exact_05_amd.build``.  The library is written
next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["api.cpp", "fa_fwd.hip", "fa_fwd_wide.hip", "fa_fwd_pipe.hip", "fa_fwd_f32.hip", "fa_fwd_fp8.hip",
           "fa_quant.hip", "fa_bwd.hip", "fa_decode.hip"]
# Extra flags per source.  fa_fwd_wide.hip and fa_fwd_pipe.hip keep their
# MFMA accumulators in VGPRs (VGPR form): their registers then fit two waves
# per SIMD with no copies between the VGPR and AGPR files.  The forward
# kernels also assume no NaN operands, which lets a row maximum be v_max3_f32
# chains without canonicalising every MFMA result first (fwd_wide: 1-2% at
# d = 256).
SOURCE_FLAGS = {"fa_fwd_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
                "fa_fwd_pipe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
                "fa_fwd_fp8.hip": ["-fno-honor-nans"]}
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled: hipcc -O3 would otherwise form
# v_pk_{add,mul,fma}_f32 from ordinary float code.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libfa.so")
    noise = [ln for ln in (r.stdout + r.stderr).splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln]
    if verbose and noise:
        print("\n".join(noise))


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source to an object (in parallel), then link libfa.so."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out_tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmp:
        objs, jobs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [hipcc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), "-I", os.path.join(ROOT, "include"),
                   "-I", CSRC, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
            objs.append(obj)
            jobs.append(cmd)
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
            list(ex.map(lambda c: _run(c, verbose), jobs))
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp], verbose)
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
