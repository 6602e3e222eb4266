"""Pins of the grouped-K/V oracle (oracle.attention_gqa): the K/V head map,
the reduction to ordinary attention, and a brute-force case.  Multi-query
attention is named on "FlashAttention (HI)" (section on development and
further research: FlashAttention-2 extends to multi-query architectures);
grouping consecutive query heads around each K/V head is the reading used
(one K/V head for all query heads when Hkv = 1)."""
import math

import numpy as np
import pytest

from oracle import oracle


def test_head_map():
    # the reading: consecutive query heads share a K/V head
    assert list(oracle.gqa_kv_index(6, 2)) == [0, 0, 0, 1, 1, 1]
    assert list(oracle.gqa_kv_index(6, 3)) == [0, 0, 1, 1, 2, 2]
    assert list(oracle.gqa_kv_index(4, 1)) == [0, 0, 0, 0]
    assert list(oracle.gqa_kv_index(4, 4)) == [0, 1, 2, 3]
    for bad in (0, 3, 5, 8):
        with pytest.raises(ValueError):
            oracle.gqa_kv_index(4, bad)


@pytest.mark.parametrize("causal", [0, 1])
def test_equal_head_counts_is_ordinary_attention(causal):
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((2, 3, 37, 64)) for _ in range(3))
    o1, l1 = oracle.attention_gqa(q, k, v, causal, 0.125)
    o2, l2 = oracle.attention(q, k, v, causal, 0.125)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("causal", [0, 1])
def test_identical_queries_group_outputs(causal):
    # every query head equal, K/V heads distinct: outputs agree inside a
    # group and differ across groups (a map by h % Hkv would pair heads 0, 2, 4)
    rng = np.random.default_rng(12)
    q1 = rng.standard_normal((1, 1, 20, 64))
    q = np.repeat(q1, 6, axis=1)
    k, v = (rng.standard_normal((1, 2, 20, 64)) for _ in range(2))
    o, lse = oracle.attention_gqa(q, k, v, causal, 0.3)
    for h in (1, 2):
        assert np.array_equal(o[:, h], o[:, 0]) and np.array_equal(lse[:, h], lse[:, 0])
    for h in (4, 5):
        assert np.array_equal(o[:, h], o[:, 3])
    assert not np.allclose(o[:, 0], o[:, 3])
    # and each group is ordinary attention with its own K/V head
    for g in range(2):
        og, lg = oracle.attention(q1, k[:, g:g + 1], v[:, g:g + 1], causal, 0.3)
        assert np.array_equal(o[:, 3 * g], og[:, 0]) and np.array_equal(lse[:, 3 * g], lg[:, 0])


def test_brute_force_two_heads_one_kv():
    # H = 2 query heads, one K/V head, N = 2 keys, d = 64 with two non-zero
    # coordinates: softmax written out by hand
    q = np.zeros((1, 2, 2, 64)); k = np.zeros((1, 1, 2, 64)); v = np.zeros((1, 1, 2, 64))
    q[0, 0, 0, 0], q[0, 0, 1, 1] = 1.0, 2.0
    q[0, 1, 0, 0], q[0, 1, 1, 0] = -1.0, 0.5
    k[0, 0, 0, 0], k[0, 0, 1, 1] = 2.0, 1.0
    v[0, 0, 0, 5], v[0, 0, 1, 5] = 3.0, -1.0
    o, lse = oracle.attention_gqa(q, k, v, 0, 0.5)
    for h in range(2):
        for i in range(2):
            s = [0.5 * float(q[0, h, i] @ k[0, 0, j]) for j in range(2)]
            z = math.exp(s[0]) + math.exp(s[1])
            want = (math.exp(s[0]) * 3.0 + math.exp(s[1]) * -1.0) / z
            assert abs(o[0, h, i, 5] - want) < 1e-14
            assert abs(lse[0, h, i] - math.log(z)) < 1e-14
