"""Pins for the fp64 CPU oracle (no GPU).

The oracle is the plain definition of exact attention: the single formula the
pages print, softmax(Q K^T / sqrt(d_k)) V ("FlashAttention (HI)" and
"FlashAttention (TL)", section on the problems of standard attention), with
the causal mask named among the fused operations (same pages, section on
combining all operations into one kernel) and the per-row logsumexp.  None of
the tests below re-types the oracle's two-pass formula: each pins it to
something else the pages or the mathematics fix — a 50-digit brute force that
takes another algebraic route, closed forms, invariants and special cases.
"""
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# 1. Brute force at N <= 8 in 50-digit decimal arithmetic.  Softmax is taken
#    as p_ij = 1 / sum_k exp(s_ik - s_ij) (no running max, no division of a
#    sum by a sum) and lse_i = ln(sum_j exp(s_ij)) directly.
# ---------------------------------------------------------------------------
def _decimal_attention(q, k, v, causal, scale):
    getcontext().prec = 50
    N, d = q.shape
    D = lambda x: Decimal(float(x))  # exact conversion of a binary64 value
    sc = D(scale)
    s = [[sc * sum(D(q[i, c]) * D(k[j, c]) for c in range(d)) for j in range(N)]
         for i in range(N)]
    o = np.zeros((N, d))
    lse = np.zeros(N)
    for i in range(N):
        vis = [j for j in range(N) if (not causal) or j <= i]
        lse[i] = float(sum((s[i][j]).exp() for j in vis).ln())
        for c in range(d):
            acc = Decimal(0)
            for j in vis:
                p = Decimal(1) / sum((s[i][t] - s[i][j]).exp() for t in vis)
                acc += p * D(v[j, c])
            o[i, c] = float(acc)
    return o, lse


@pytest.mark.parametrize("N,d", [(1, 1), (2, 3), (5, 4), (8, 8), (7, 2)])
@pytest.mark.parametrize("causal", [0, 1])
def test_decimal_brute_force(N, d, causal):
    for seed in range(2):
        q = _rand((1, 1, N, d), 10 * N + d + seed, 1.5)
        k = _rand((1, 1, N, d), 20 * N + d + seed, 1.5)
        v = _rand((1, 1, N, d), 30 * N + d + seed)
        scale = 1.0 / math.sqrt(d)
        o, lse = oracle.attention(q, k, v, causal, scale)
        o_ref, lse_ref = _decimal_attention(q[0, 0], k[0, 0], v[0, 0], causal, scale)
        np.testing.assert_allclose(o[0, 0], o_ref, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[0, 0], lse_ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# 2. Rows of P are probability vectors: with d = N and V = I, row i of O is
#    row i of P.  It must be >= 0, sum to 1, and vanish above the diagonal
#    when causal.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("N", [1, 4, 33, 64])
def test_rows_of_p_sum_to_one(N, causal):
    q = _rand((2, 1, N, N), 1, 2.0)
    k = _rand((2, 1, N, N), 2, 2.0)
    v = np.broadcast_to(np.eye(N), (2, 1, N, N)).copy()
    o, _ = oracle.attention(q, k, v, causal, 0.7)
    p = o  # O = P V = P
    assert (p >= 0).all()
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-14 * N)
    if causal:
        upper = np.triu(np.ones((N, N), bool), 1)
        assert np.all(p[..., upper] == 0.0)


# ---------------------------------------------------------------------------
# 3. Convex combination: constant V rows give that constant back.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [0, 1])
def test_constant_v(causal):
    B, H, N, d = 2, 3, 37, 16
    q, k = _rand((B, H, N, d), 3), _rand((B, H, N, d), 4)
    c = _rand((B, H, 1, d), 5)
    v = np.broadcast_to(c, (B, H, N, d)).copy()
    o, _ = oracle.attention(q, k, v, causal, 0.25)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# 4. The online recurrence (what the tiled kernel computes) equals the
#    definition: processing keys in chunks with a running max m and running
#    sum l, rescaling the partial output by exp(m_old - m_new), gives the same
#    O and logsumexp ("online softmax" section of the FlashAttention pages).
#    Done both in base e and in the base-2 form the GPU uses.
# ---------------------------------------------------------------------------
def _online_rows(q, k, v, causal, scale, chunk, base2):
    N, d = q.shape
    o = np.zeros((N, d))
    lse = np.zeros(N)
    L2E = 1.0 / math.log(2.0)
    for i in range(N):
        m, l, acc = -1e300, 0.0, np.zeros(d)
        last = i + 1 if causal else N
        for j0 in range(0, last, chunk):
            js = range(j0, min(j0 + chunk, last))
            s = np.array([scale * float(np.dot(q[i], k[j])) for j in js])
            if base2:
                t = s * L2E
                m_new = max(m, t.max())
                alpha = 2.0 ** (m - m_new)
                p = 2.0 ** (t - m_new)
            else:
                m_new = max(m, s.max())
                alpha = math.exp(m - m_new)
                p = np.exp(s - m_new)
            l = alpha * l + p.sum()
            acc = alpha * acc + p @ v[list(js)]
            m = m_new
        o[i] = acc / l
        lse[i] = (m + math.log2(l)) * math.log(2.0) if base2 else m + math.log(l)
    return o, lse


@pytest.mark.parametrize("chunk", [1, 2, 3, 7, 23])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("base2", [False, True])
def test_two_pass_equals_online(chunk, causal, base2):
    N, d = 23, 5
    q, k, v = _rand((1, 1, N, d), 6, 2.0), _rand((1, 1, N, d), 7, 2.0), _rand((1, 1, N, d), 8)
    o, lse = oracle.attention(q, k, v, causal, 0.6)
    o2, lse2 = _online_rows(q[0, 0], k[0, 0], v[0, 0], causal, 0.6, chunk, base2)
    np.testing.assert_allclose(o[0, 0], o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], lse2, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# 5. Key order does not matter without a mask: permuting K and V rows jointly
#    leaves O and the logsumexp unchanged.
# ---------------------------------------------------------------------------
def test_joint_key_permutation_noncausal():
    B, H, N, d = 1, 2, 50, 8
    q, k, v = _rand((B, H, N, d), 9), _rand((B, H, N, d), 10), _rand((B, H, N, d), 11)
    perm = np.random.default_rng(12).permutation(N)
    o1, l1 = oracle.attention(q, k, v, 0, 0.35)
    o2, l2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0, 0.35)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# 6. Closed form at Q = 0: every visible key gets weight 1/|A_i|, so
#    lse_i = ln N (ln(i+1) causal) and O_i is the mean of the visible V rows.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [0, 1])
def test_zero_query_closed_form(causal):
    B, H, N, d = 1, 1, 40, 6
    q = np.zeros((B, H, N, d))
    k, v = _rand((B, H, N, d), 13, 3.0), _rand((B, H, N, d), 14)
    o, lse = oracle.attention(q, k, v, causal, 1.0)
    for i in range(N):
        n = i + 1 if causal else N
        np.testing.assert_allclose(lse[0, 0, i], math.log(n), rtol=0, atol=1e-14)
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n].mean(0), rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# 7. Causal boundary: query 0 sees only key 0, so O_0 = v_0 and
#    lse_0 = scale * q_0 . k_0.
# ---------------------------------------------------------------------------
def test_causal_row_zero():
    B, H, N, d = 2, 2, 9, 7
    q, k, v = _rand((B, H, N, d), 15), _rand((B, H, N, d), 16), _rand((B, H, N, d), 17)
    o, lse = oracle.attention(q, k, v, 1, 0.45)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    dots = (q[:, :, 0] * k[:, :, 0]).sum(-1)
    np.testing.assert_allclose(lse[:, :, 0], 0.45 * dots, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------------
# 8. Shift invariance: appending a column 1 to every query and a column c to
#    every key adds scale*c to every score — the softmax is unchanged and the
#    logsumexp moves by scale*c.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [0, 1])
def test_shift_invariance(causal):
    B, H, N, d = 1, 2, 31, 5
    q, k, v = _rand((B, H, N, d), 18), _rand((B, H, N, d), 19), _rand((B, H, N, d), 20)
    c, scale = 3.25, 0.5
    q2 = np.concatenate([q, np.ones((B, H, N, 1))], -1)
    k2 = np.concatenate([k, np.full((B, H, N, 1), c)], -1)
    o1, l1 = oracle.attention(q, k, v, causal, scale)
    # widen v to the new width with a zero column, then drop it again
    v2 = np.concatenate([v, np.zeros((B, H, N, 1))], -1)
    o2, l2 = oracle.attention(q2, k2, v2, causal, scale)
    np.testing.assert_allclose(o2[..., :d], o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1 + scale * c, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# 9. Worked two-key case (a closed form of the formula, stored under golden/):
#    d = 1, N = 2, scale = 1, q = 1, k = (0, ln 2)  ->  p = (1/3, 2/3).
# ---------------------------------------------------------------------------
def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                key, val = line.split("=", 1)
                vals[key.strip()] = [float(x) for x in val.split()]
    return vals


def test_worked_two_key_case():
    g = _read_golden("two_key_closed_form.txt")
    N = 2
    q = np.array(g["q"]).reshape(1, 1, N, 1)
    k = np.array(g["k"]).reshape(1, 1, N, 1)
    v = np.array(g["v"]).reshape(1, 1, N, 1)
    o, lse = oracle.attention(q, k, v, 0, g["scale"][0])
    np.testing.assert_allclose(o.reshape(-1), g["o"], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(lse.reshape(-1), g["lse"], rtol=1e-15, atol=1e-15)


# ---------------------------------------------------------------------------
# 10. Numerical range: scores near 1e3 must not overflow; one key that
#     dominates by a margin of 200 takes all the weight (exp(-200) < 1e-86).
# ---------------------------------------------------------------------------
def test_large_scores_dominant_key():
    N, d = 16, 4
    q = np.zeros((1, 1, N, d)); q[..., 0] = 1.0
    k = np.zeros((1, 1, N, d)); k[..., 0] = 800.0; k[0, 0, 11, 0] = 1000.0
    v = _rand((1, 1, N, d), 21)
    o, lse = oracle.attention(q, k, v, 0, 1.0)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, 11], (N, d)), atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], 1000.0, rtol=1e-15)


# ---------------------------------------------------------------------------
# 11. Scale moves into Q: attention(q, k, v, scale) == attention(scale*q, k, v, 1)
#     for scale a power of two (so scale*q is exact).
# ---------------------------------------------------------------------------
def test_scale_moves_into_query():
    B, H, N, d = 1, 1, 20, 8
    q, k, v = _rand((B, H, N, d), 22), _rand((B, H, N, d), 23), _rand((B, H, N, d), 24)
    o1, l1 = oracle.attention(q, k, v, 1, 0.125)
    o2, l2 = oracle.attention(q * 0.125, k, v, 1, 1.0)
    np.testing.assert_allclose(o1, o2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# 12. Heads and batches are independent: the oracle over [B,H] equals the
#     oracle run on each head alone, and the selected-rows entry point equals
#     the corresponding rows of the full call.
# ---------------------------------------------------------------------------
def test_heads_independent_and_rows_api():
    B, H, N, d = 2, 3, 17, 4
    q, k, v = _rand((B, H, N, d), 25), _rand((B, H, N, d), 26), _rand((B, H, N, d), 27)
    o, lse = oracle.attention(q, k, v, 1, 0.3)
    for b in range(B):
        for h in range(H):
            o1, l1 = oracle.attention(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                      v[b:b + 1, h:h + 1], 1, 0.3)
            np.testing.assert_array_equal(o1[0, 0], o[b, h])
            np.testing.assert_array_equal(l1[0, 0], lse[b, h])
    rows = np.array([0, 5, 16, 17, 40, B * H * N - 1])
    orow, lrow = oracle.attention_rows(q, k, v, 1, 0.3, rows)
    np.testing.assert_array_equal(orow, o.reshape(-1, d)[rows])
    np.testing.assert_array_equal(lrow, lse.reshape(-1)[rows])


def test_bad_arguments_rejected():
    lib = oracle.load()
    q = np.zeros((1, 1, 2, 2))
    with pytest.raises(RuntimeError):
        oracle.attention_rows(q, q, q, 0, 1.0, [4])  # row index out of range
