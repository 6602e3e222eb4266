"""fp64 CPU oracle of attention over a key/value cache — TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module; the GPU library never calls it and the two share
no code.

The workload is the KV-cache inference named on "FlashAttention (HI)"
(section on specialised solutions: FlashInfer and streaming generation with a
KV cache): a few new queries per head (Nq, e.g. one decoded token) attend to a
long cache of Nkv >= Nq keys and values.  The result is the same formula as
everywhere on the pages, O = softmax(scale * Q K^T) V ("FlashAttention (HI)" /
"(TL)", section on the problems of standard attention), now with Q of Nq rows
and K, V of Nkv rows.  Causal masking in this setting (the reading used
here): the Nq queries are the LAST Nq positions of the sequence, so query i
(0-based) sees cache keys j <= Nkv - Nq + i; Nq = 1 sees the whole cache.
K/V heads may be shared by groups of consecutive query heads, as in
oracle.gqa_kv_index.  Matrix products are numpy's; nothing is blocked.
"""
from __future__ import annotations

import numpy as np

from .oracle import _f64, gqa_kv_index


def attention_kvcache(q, k, v, causal: bool, scale: float):
    """q [B, H, Nq, d]; k, v [B, Hkv, Nkv, d] with Hkv | H and Nq <= Nkv.
    Returns (o [B, H, Nq, d], lse [B, H, Nq]) in fp64, lse the natural-log
    logsumexp of each masked, scaled score row."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or k.shape[0] != q.shape[0] \
            or k.shape[3] != q.shape[3]:
        raise ValueError("q must be [B, H, Nq, d] and k, v one [B, Hkv, Nkv, d] shape")
    B, H, Nq, d = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    if Nq > Nkv:
        raise ValueError("the cache must hold at least as many keys as there are queries")
    kv_of = gqa_kv_index(H, Hkv)
    o = np.empty((B, H, Nq, d))
    lse = np.empty((B, H, Nq))
    vis = np.arange(Nkv)[None, :] <= (Nkv - Nq + np.arange(Nq))[:, None]
    for b in range(B):
        for h in range(H):
            g = kv_of[h]
            s = scale * (q[b, h] @ k[b, g].T)
            if causal:
                s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            l = e.sum(axis=1, keepdims=True)
            o[b, h] = (e / l) @ v[b, g]
            lse[b, h] = (m + np.log(l))[:, 0]
    return o, lse
