"""Pins of the KV-cache oracle (oracle.attention_kvcache), no GPU.

Each check ties it to something other than its own code: the separate C
forward oracle (equal lengths; the last rows of a causal prefill), a
50-digit brute force, a closed form, and the logsumexp merge identity that
split-KV evaluation relies on (attention over a cache cut in two parts equals
the two partial results weighted by exp(lse_part - lse)).
"""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("causal", [0, 1])
def test_equal_lengths_match_the_c_oracle(causal):
    q, k, v = _rand((2, 3, 45, 16), 1), _rand((2, 3, 45, 16), 2), _rand((2, 3, 45, 16), 3)
    o, lse = oracle.attention_kvcache(q, k, v, causal, 0.3)
    o2, lse2 = oracle.attention(q, k, v, causal, 0.3)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("Nq", [1, 3, 16])
def test_decoded_rows_are_the_last_rows_of_a_causal_prefill(Nq):
    # the reading of causal decoding: the new queries are the sequence's last
    # Nq positions, so they must reproduce the last Nq rows of causal attention
    # over the whole sequence (C oracle)
    N, d = 70, 32
    q, k, v = _rand((1, 2, N, d), 4, 1.5), _rand((1, 2, N, d), 5, 1.5), _rand((1, 2, N, d), 6)
    o_full, lse_full = oracle.attention(q, k, v, 1, 1 / math.sqrt(d))
    o, lse = oracle.attention_kvcache(q[:, :, N - Nq:], k, v, 1, 1 / math.sqrt(d))
    np.testing.assert_allclose(o, o_full[:, :, N - Nq:], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_full[:, :, N - Nq:], rtol=1e-13, atol=1e-13)


def test_single_query_sees_the_whole_cache_either_way():
    q, k, v = _rand((1, 4, 1, 8), 7), _rand((1, 2, 33, 8), 8), _rand((1, 2, 33, 8), 9)
    a = oracle.attention_kvcache(q, k, v, 0, 0.5)
    b = oracle.attention_kvcache(q, k, v, 1, 0.5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_identical_keys_average_the_values():
    # equal scores: O = mean of the visible values, lse = ln(count) + score
    Nkv, Nq, d = 20, 4, 8
    k = np.broadcast_to(_rand((1, 1, 1, d), 10), (1, 1, Nkv, d)).copy()
    q, v = _rand((1, 1, Nq, d), 11), _rand((1, 1, Nkv, d), 12)
    for causal in (0, 1):
        o, lse = oracle.attention_kvcache(q, k, v, causal, 0.7)
        for i in range(Nq):
            n = Nkv - Nq + i + 1 if causal else Nkv
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n].mean(axis=0), rtol=1e-12, atol=1e-13)
            s = 0.7 * float(q[0, 0, i] @ k[0, 0, 0])
            assert abs(lse[0, 0, i] - (math.log(n) + s)) < 1e-12


@pytest.mark.parametrize("causal", [0, 1])
def test_decimal_brute_force(causal):
    getcontext().prec = 50
    Nq, Nkv, d = 3, 7, 3
    q, k, v = _rand((1, 1, Nq, d), 13, 1.5), _rand((1, 1, Nkv, d), 14, 1.5), _rand((1, 1, Nkv, d), 15)
    o, lse = oracle.attention_kvcache(q, k, v, causal, 0.9)
    D = lambda x: Decimal(float(x))
    for i in range(Nq):
        vis = [j for j in range(Nkv) if not causal or j <= Nkv - Nq + i]
        s = {j: D(0.9) * sum(D(q[0, 0, i, c]) * D(k[0, 0, j, c]) for c in range(d)) for j in vis}
        z = sum(x.exp() for x in s.values())
        assert abs(float(z.ln()) - lse[0, 0, i]) < 1e-13
        for c in range(d):
            want = sum(s[j].exp() / z * D(v[0, 0, j, c]) for j in vis)
            assert abs(float(want) - o[0, 0, i, c]) < 1e-13


@pytest.mark.parametrize("cut", [1, 17, 39])
def test_split_merge_identity(cut):
    # attention over the cache [0, Nkv) from attention over [0, cut) and
    # [cut, Nkv): lse = ln(e^lse1 + e^lse2), O = e^(lse1-lse) O1 + e^(lse2-lse) O2
    Nkv, d = 40, 16
    q, k, v = _rand((2, 4, 1, d), 16), _rand((2, 2, Nkv, d), 17), _rand((2, 2, Nkv, d), 18)
    o, lse = oracle.attention_kvcache(q, k, v, 0, 0.25)
    o1, l1 = oracle.attention_kvcache(q, k[:, :, :cut], v[:, :, :cut], 0, 0.25)
    o2, l2 = oracle.attention_kvcache(q, k[:, :, cut:], v[:, :, cut:], 0, 0.25)
    lm = np.logaddexp(l1, l2)
    om = np.exp(l1 - lm)[..., None] * o1 + np.exp(l2 - lm)[..., None] * o2
    np.testing.assert_allclose(lse, lm, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o, om, rtol=1e-12, atol=1e-13)


def test_shared_heads_match_the_grouped_oracle():
    q, k, v = _rand((2, 6, 30, 16), 19), _rand((2, 3, 30, 16), 20), _rand((2, 3, 30, 16), 21)
    for causal in (0, 1):
        o, lse = oracle.attention_kvcache(q, k, v, causal, 0.4)
        o2, lse2 = oracle.attention_gqa(q, k, v, causal, 0.4)
        np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, lse2, rtol=1e-13, atol=1e-13)


def test_shape_errors():
    with pytest.raises(ValueError):
        oracle.attention_kvcache(np.zeros((1, 1, 5, 8)), np.zeros((1, 1, 4, 8)), np.zeros((1, 1, 4, 8)), 0, 1.0)
    with pytest.raises(ValueError):
        oracle.attention_kvcache(np.zeros((1, 4, 1, 8)), np.zeros((1, 3, 4, 8)), np.zeros((1, 3, 4, 8)), 0, 1.0)
