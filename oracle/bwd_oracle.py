"""fp64 CPU oracle of the attention backward pass — TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module; the GPU library never calls it and the two share
no code.

The pages describe the forward pass only: the one formula O = softmax(S) V
with S = scale * Q K^T ("FlashAttention (HI)" / "FlashAttention (TL)",
section on the problems of standard attention), the causal mask among the
fused operations (same pages, section on combining everything into one
kernel), and training speed-ups that need its gradient.  The gradient is
therefore derived here by differentiating that formula; the loss seen by the
inputs is L = sum(dO * O) for a given upstream gradient dO, and for one
(batch, head) with P = softmax(S) row by row (hidden keys have P = 0):

    dV = P^T dO
    dP = dO V^T
    dS_ij = P_ij (dP_ij - D_i),   D_i = sum_j P_ij dP_ij = dO_i . O_i
    dQ = scale * dS K
    dK = scale * dS^T Q

(softmax Jacobian: d p_j / d s_l = p_j (delta_jl - p_l)).  When K/V heads are
shared by a group of query heads, K and V enter every head of the group, so
their gradients are the sums over the group.  Matrix products are numpy's
(a library primitive); nothing is blocked or reordered.
"""
from __future__ import annotations

import numpy as np

from .oracle import _f64, gqa_kv_index


def _head_grads(q, k, v, do, causal: bool, scale: float):
    """Gradients of one head: q, k, v, do [N, d] fp64 -> dq, dk, dv, delta."""
    N = q.shape[0]
    s = scale * (q @ k.T)
    if causal:
        s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    o = p @ v
    dv = p.T @ do
    dp = do @ v.T
    delta = (do * o).sum(axis=1)
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv, delta


def attention_bwd(q, k, v, dout, causal: bool, scale: float, heads=None):
    """Backward pass of exact attention in fp64.

    q, dout: [B, H, N, d]; k, v: [B, Hkv, N, d] with Hkv dividing H (query head
    h uses K/V head h // (H // Hkv)).  Returns (dq [B,H,N,d], dk [B,Hkv,N,d],
    dv [B,Hkv,N,d], delta [B,H,N]) with delta_i = dO_i . O_i.

    heads: optional iterable of flat K/V head indices b*Hkv + g; only those
    K/V heads (and the query heads of their groups) are computed, the rest of
    every output is NaN.  Used to check sampled heads of large workloads.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    if q.ndim != 4 or k.ndim != 4 or q.shape != do.shape or k.shape != v.shape \
            or k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:]:
        raise ValueError("q, dout must be [B, H, N, d] and k, v one [B, Hkv, N, d] shape")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    kv_of = gqa_kv_index(H, Hkv)
    full = heads is None
    fill = 0.0 if full else np.nan
    dq = np.full(q.shape, fill)
    dk = np.full(k.shape, fill)
    dv = np.full(v.shape, fill)
    delta = np.full((B, H, N), fill)
    todo = range(B * Hkv) if full else sorted(set(int(x) for x in heads))
    for flat in todo:
        b, g = divmod(flat, Hkv)
        dk[b, g] = 0.0
        dv[b, g] = 0.0
        for h in np.nonzero(kv_of == g)[0]:
            gq, gk, gv, dl = _head_grads(q[b, h], k[b, g], v[b, g], do[b, h], causal, scale)
            dq[b, h] = gq
            dk[b, g] += gk
            dv[b, g] += gv
            delta[b, h] = dl
    return dq, dk, dv, delta
