"""Accuracy gates between the GPU output and the fp64 oracle (test helpers).

O (fp16/bf16/fp32 outputs): elementwise |O_gpu - O_ref| <= 1e-2 + ulp_out(O_ref)/2.
  The 1e-2 bounds the computation error; the half-ulp term is the rounding of
  a perfect result to the output dtype, which alone exceeds 1e-2 for bf16 once
  |O| >= 4 (bf16 spacing is 2^-5 there).
LSE: |LSE_gpu - LSE_ref| <= 1e-3.
Any NaN or Inf fails.  All differences are taken in fp64 after exact widening.
"""
from __future__ import annotations

import numpy as np
import torch

O_ABS_TOL = 1e-2
LSE_ABS_TOL = 1e-3

_PREC = {"bf16": (8, -126), "f16": (11, -14), "f32": (24, -126)}  # (precision bits, emin)


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the output dtype's numbers at |x| (normal or subnormal range)."""
    p, emin = _PREC[dtype]
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 2.0 ** emin)))
    e = np.maximum(e, emin)
    return 2.0 ** (e - (p - 1))


def widen(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, np.float64)


def check(o_gpu, lse_gpu, o_ref, lse_ref, out_dtype: str, what: str = ""):
    """Assert the gates; return a dict of the measured errors."""
    o_gpu, lse_gpu = widen(o_gpu), widen(lse_gpu)
    o_ref, lse_ref = np.asarray(o_ref, np.float64), np.asarray(lse_ref, np.float64)
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite O"
    assert np.isfinite(lse_gpu).all(), f"{what}: non-finite LSE"
    err = np.abs(o_gpu - o_ref)
    gate = O_ABS_TOL + 0.5 * ulp(o_ref, out_dtype)
    lse_err = np.abs(lse_gpu - lse_ref)
    stats = {
        "o_max_abs": float(err.max(initial=0.0)),
        "o_excess": float((err - gate).max(initial=-1.0)),
        "lse_max_abs": float(lse_err.max(initial=0.0)),
        "n_big": int((np.abs(o_ref) >= 4).sum()),
    }
    bad = err > gate
    if bad.any():
        idx = np.unravel_index(np.argmax(err - gate), err.shape)
        raise AssertionError(f"{what}: O gate failed at {idx}: gpu={o_gpu[idx]!r} "
                             f"ref={o_ref[idx]!r} ({int(bad.sum())} elements) {stats}")
    assert (lse_err <= LSE_ABS_TOL).all(), f"{what}: LSE gate failed {stats}"
    return stats
