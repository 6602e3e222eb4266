"""Pins of the backward-pass oracle (oracle.attention_bwd), no GPU.

The pages give no backward pass; its definition is the derivative of the
forward formula ("FlashAttention (HI)" / "(TL)", section on the problems of
standard attention) for the loss L = sum(dO * O).  Nothing below re-types the
oracle's chain-rule formulas: each check pins them to something else —
central finite differences of the (separate, C) forward oracle, closed forms,
invariants that follow from the softmax's shift invariance and from the
forward being linear in V, and torch's automatic differentiation.
Every check is a function of the gradient routine so that
test_bwd_oracle_mutants.py can run the same battery against planted mistakes.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _loss(q, k, v, do, causal, scale):
    """L = sum(dO * O) with O from the forward oracle (K/V heads repeated for groups)."""
    o, _ = oracle.attention_gqa(q, k, v, causal, scale)
    return float((do * o).sum())


# 1. Central finite differences of the forward oracle, every input element.
def pin_finite_differences(bwd, causal, H=2, Hkv=1, N=5, d=3, seed=0):
    q = _rand((1, H, N, d), seed + 1, 1.2)
    k = _rand((1, Hkv, N, d), seed + 2, 1.2)
    v = _rand((1, Hkv, N, d), seed + 3)
    do = _rand((1, H, N, d), seed + 4)
    scale = 0.7
    dq, dk, dv, _ = bwd(q, k, v, do, causal, scale)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            keep = x[idx]
            x[idx] = keep + h
            lp = _loss(q, k, v, do, causal, scale)
            x[idx] = keep - h
            lm = _loss(q, k, v, do, causal, scale)
            x[idx] = keep
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


# 2. One key per row: N = 1 gives O = V, so dV = dO and no score matters.
def pin_single_key(bwd):
    q, k, v, do = (_rand((2, 3, 1, 8), s) for s in range(4))
    for causal in (0, 1):
        dq, dk, dv, delta = bwd(q, k, v, do, causal, 0.9)
        np.testing.assert_allclose(dv, do, rtol=0, atol=1e-15)
        # dS = 1 * (dO.v - dO.v): zero up to the two dot products' rounding
        assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
        np.testing.assert_allclose(delta, (do * v).sum(-1), rtol=1e-14, atol=1e-14)


# 3. Zero queries: every visible key gets weight 1 / (#visible).  Then
#    dV_j = sum over rows i that see j of dO_i / (#visible in row i), and
#    dK = scale * dS^T Q = 0.  Causal row 0 sees one key, so dQ_0 = 0.
def pin_zero_queries(bwd):
    N, d = 9, 4
    q = np.zeros((1, 1, N, d))
    k, v, do = _rand((1, 1, N, d), 7), _rand((1, 1, N, d), 8), _rand((1, 1, N, d), 9)
    for causal in (0, 1):
        dq, dk, dv, _ = bwd(q, k, v, do, causal, 0.5)
        want = np.zeros((N, d))
        for i in range(N):
            vis = range(i + 1) if causal else range(N)
            for j in vis:
                want[j] += do[0, 0, i] / len(vis)
        np.testing.assert_allclose(dv[0, 0], want, rtol=1e-13, atol=1e-14)
        assert np.abs(dk).max() < 1e-14
        if causal:
            assert np.abs(dq[0, 0, 0]).max() < 1e-15


# 4. Invariants at random inputs.
#  (a) Adding one vector to every key shifts each score row by a constant,
#      which softmax ignores: the keys' gradients sum to zero.
#  (b) L depends on scale and Q K^T only through scale * q_i . k_j, so
#      sum_i q_i . dQ_i = sum_j k_j . dK_j = scale * dL/dscale (checked
#      against a finite difference in the scale).
#  (c) O is linear in V: sum_j v_j . dV_j = sum_i dO_i . O_i = sum_i delta_i.
def pin_invariants(bwd, causal):
    B, H, Hkv, N, d = 1, 4, 2, 40, 16
    q, k = _rand((B, H, N, d), 11, 1.3), _rand((B, Hkv, N, d), 12, 1.3)
    v, do = _rand((B, Hkv, N, d), 13), _rand((B, H, N, d), 14)
    scale = 0.3
    dq, dk, dv, delta = bwd(q, k, v, do, causal, scale)
    assert np.abs(dk.sum(axis=2)).max() < 1e-11
    qdq = (q * dq).sum()
    kdk = (k * dk).sum()
    assert abs(qdq - kdk) < 1e-10 * (1 + abs(qdq))
    h = 1e-6
    dl_dscale = (_loss(q, k, v, do, causal, scale + h) - _loss(q, k, v, do, causal, scale - h)) / (2 * h)
    assert abs(qdq - scale * dl_dscale) < 1e-6 * (1 + abs(qdq))
    o, _ = oracle.attention_gqa(q, k, v, causal, scale)
    np.testing.assert_allclose(delta, (do * o).sum(-1), rtol=1e-12, atol=1e-12)
    assert abs((v * dv).sum() - delta.sum()) < 1e-10 * (1 + abs(delta.sum()))


# 5. Shared K/V heads: K and V enter every head of a group, so their gradient
#    is the sum of the per-head gradients computed with K/V repeated.
def pin_groups_sum(bwd, causal):
    B, H, Hkv, N, d = 2, 6, 2, 17, 8
    q, k = _rand((B, H, N, d), 21), _rand((B, Hkv, N, d), 22)
    v, do = _rand((B, Hkv, N, d), 23), _rand((B, H, N, d), 24)
    idx = oracle.gqa_kv_index(H, Hkv)
    dq, dk, dv, _ = bwd(q, k, v, do, causal, 0.4)
    dq1, dk1, dv1, _ = bwd(q, k[:, idx].copy(), v[:, idx].copy(), do, causal, 0.4)
    np.testing.assert_allclose(dq, dq1, rtol=1e-13, atol=1e-13)
    for g in range(Hkv):
        np.testing.assert_allclose(dk[:, g], dk1[:, idx == g].sum(axis=1), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dv[:, g], dv1[:, idx == g].sum(axis=1), rtol=1e-12, atol=1e-12)


# 6. Automatic differentiation (torch, fp64, CPU) of the plain forward formula.
def pin_autograd(bwd, causal):
    B, H, N, d = 1, 2, 37, 8
    q, k, v, do = (_rand((B, H, N, d), 31 + s) for s in range(4))
    scale = 1 / math.sqrt(d)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = scale * tq @ tk.transpose(-1, -2)
    if causal:
        s = s.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    o.backward(torch.tensor(do))
    dq, dk, dv, _ = bwd(q, k, v, do, causal, scale)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-11, atol=1e-12)


# 7. Sampled heads agree with the full computation and leave the rest NaN.
def pin_sampled_heads(bwd):
    B, H, Hkv, N, d = 2, 4, 2, 12, 8
    q, k = _rand((B, H, N, d), 41), _rand((B, Hkv, N, d), 42)
    v, do = _rand((B, Hkv, N, d), 43), _rand((B, H, N, d), 44)
    full = bwd(q, k, v, do, 1, 0.5)
    part = bwd(q, k, v, do, 1, 0.5, heads=[1, 2])
    # K/V head 1 = (b 0, g 1): query heads 2, 3 of batch 0; head 2 = (b 1, g 0)
    np.testing.assert_array_equal(part[1][0, 1], full[1][0, 1])
    np.testing.assert_array_equal(part[2][1, 0], full[2][1, 0])
    np.testing.assert_array_equal(part[0][0, 2:], full[0][0, 2:])
    np.testing.assert_array_equal(part[0][1, :2], full[0][1, :2])
    assert np.isnan(part[1][0, 0]).all() and np.isnan(part[0][0, :2]).all()


BWD = oracle.attention_bwd


@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("H,Hkv", [(1, 1), (2, 1)])
def test_finite_differences(causal, H, Hkv):
    pin_finite_differences(BWD, causal, H=H, Hkv=Hkv)


def test_single_key():
    pin_single_key(BWD)


def test_zero_queries():
    pin_zero_queries(BWD)


@pytest.mark.parametrize("causal", [0, 1])
def test_invariants(causal):
    pin_invariants(BWD, causal)


@pytest.mark.parametrize("causal", [0, 1])
def test_groups_sum(causal):
    pin_groups_sum(BWD, causal)


@pytest.mark.parametrize("causal", [0, 1])
def test_autograd(causal):
    pin_autograd(BWD, causal)


def test_sampled_heads():
    pin_sampled_heads(BWD)


def test_shape_errors():
    q = np.zeros((1, 4, 8, 16))
    with pytest.raises(ValueError):
        BWD(q, np.zeros((1, 3, 8, 16)), np.zeros((1, 3, 8, 16)), q, 0, 1.0)
    with pytest.raises(ValueError):
        BWD(q, np.zeros((1, 2, 8, 16)), np.zeros((1, 2, 8, 16)), np.zeros((1, 4, 8, 8)), 0, 1.0)
