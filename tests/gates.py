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


# ---------------------------------------------------------------------------
# Backward pass.  The GPU rounds three things the fp64 gradient does not:
#  - P (relative error <= u) before dV = P^T dO;
#  - dS (relative <= u) before dQ = scale dS K and dK = scale dS^T Q;
#  - its own O (the forward's output, whose error is <= u |O| + u (P |V|)
#    per element: output rounding plus the forward's rounded P), which
#    enters D_i = dO_i . O_i and through it every dS_ij as P_ij * error(D_i);
# and then rounds each gradient to the output type (<= u |g|).  With u the
# unit roundoff of the input type, the elementwise bounds are
#   |dV err| <= u (P^T |dO|) + u |dV|
#   |dQ err| <= scale ((u |dS| + P e_D) |K|) + u |dQ|,  e_D = u |dO| . (|O| + P |V|)
#   |dK err| <= scale ((u |dS| + P e_D)^T |Q|) + u |dK|
# (shared K/V heads: sums over the group).  fp32 accumulation, exp2 and the
# forward's logsumexp add errors near 2^-20 relative; the gate is twice the
# bound plus 1e-5 of the tensor's largest magnitude.
# ---------------------------------------------------------------------------
_UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def bwd_bounds(q, k, v, do, causal, scale, dtype, heads=None):
    """Elementwise error bounds (fp64 numpy) for dq, dk, dv; heads as in
    oracle.attention_bwd (K/V heads b*Hkv + g), others left NaN."""
    u = _UNIT[dtype]
    q, k, v, do = widen(q), widen(k), widen(v), widen(do)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    grp = H // Hkv
    bq, bk, bv = (np.full(x.shape, np.nan) for x in (q, k, v))
    todo = range(B * Hkv) if heads is None else sorted(set(int(x) for x in heads))
    for flat in todo:
        b, g = divmod(flat, Hkv)
        bk[b, g] = 0.0
        bv[b, g] = 0.0
        for h in range(g * grp, (g + 1) * grp):
            s = scale * (q[b, h] @ k[b, g].T)
            if causal:
                s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o = p @ v[b, g]
            dp = do[b, h] @ v[b, g].T
            ds = p * (dp - (do[b, h] * o).sum(axis=1)[:, None])
            e_d = u * (np.abs(do[b, h]) * (np.abs(o) + p @ np.abs(v[b, g]))).sum(axis=1)
            w = u * np.abs(ds) + p * e_d[:, None]
            dq = scale * (ds @ k[b, g])
            bq[b, h] = abs(scale) * (w @ np.abs(k[b, g])) + u * np.abs(dq)
            bk[b, g] += abs(scale) * (w.T @ np.abs(q[b, h])) + u * np.abs(scale * (ds.T @ q[b, h]))
            bv[b, g] += u * (p.T @ np.abs(do[b, h])) + u * np.abs(p.T @ do[b, h])
    return bq, bk, bv


def check_bwd(grads_gpu, grads_ref, bounds, what=""):
    """Assert |gpu - ref| <= 2 bound + 1e-5 max|ref| for each of dq, dk, dv over the
    elements where the reference is defined (not NaN); return the worst error/gate ratios."""
    ratios = {}
    for name, g, r, bd in zip(("dq", "dk", "dv"), grads_gpu, grads_ref, bounds):
        g = widen(g)
        sel = ~np.isnan(r)
        assert g.shape == r.shape, (name, g.shape, r.shape)
        assert np.isfinite(g[sel]).all(), f"{what}: non-finite {name}"
        err = np.abs(g[sel] - r[sel])
        gate = 2.0 * bd[sel] + 1e-5 * np.abs(r[sel]).max(initial=0.0)
        ratio = err / np.maximum(gate, 1e-300)
        ratios[name] = float(ratio.max(initial=0.0))
        if (err > gate).any():
            i = int(np.argmax(err - gate))
            raise AssertionError(f"{what}: {name} gate failed: gpu={g[sel][i]!r} ref={r[sel][i]!r} "
                                 f"gate={gate[i]!r} ({int((err > gate).sum())} elements) {ratios}")
    return ratios
