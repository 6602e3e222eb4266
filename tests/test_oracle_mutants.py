"""The pins must catch plausible mistakes in the oracle (no GPU).

Each case below plants one mistake in a temporary copy of the oracle's C
source (a dropped term, a wrong sign or index, a transposed operand, a wrong
mask boundary), builds it with gcc, and checks that at least one of the pins
of test_oracle_pins.py, run against the mutant, fails.  Mistakes are planted
only in the oracle, only on the CPU.
"""
import math
import os
import shutil
import tempfile

import numpy as np
import pytest

import oracle
from oracle import oracle as oracle_mod

import test_oracle_pins as pins

MUTANTS = {
    "dropped_scale": ("s[j] = scale * dot;", "s[j] = dot;"),
    "causal_off_by_one": ("i + 1 < N ? i + 1 : N", "i < N ? (i > 0 ? i : 1) : N"),
    "mask_ignored": ("causal ? (i + 1 < N ? i + 1 : N) : N", "N"),
    "transposed_k": ("dot += qi[c] * kj[c];", "dot += qi[c] * k[c * N + j];"),
    "no_normalisation": ("o_row[c] /= l;", "o_row[c] /= 1.0;"),
    "lse_dropped_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "exp_sign_flipped": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "v_rows_reversed": ("const double *vj = v + j * d;",
                        "const double *vj = v + (nvis - 1 - j) * d;"),
    "query_ignores_head": ("attend_one_row(q + flat * d, kh, vh, N, d, causal, scale, i, s,\n"
                           "                               o + flat * d",
                           "attend_one_row(q + i * d, kh, vh, N, d, causal, scale, i, s,\n"
                           "                               o + flat * d"),
    "unshifted_exp": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
}


def _battery(lib):
    """Run the pins against `lib`; return the names of those that fail."""
    failures = []

    def attempt(name, fn):
        try:
            fn()
        except AssertionError:
            failures.append(name)
        except RuntimeError:
            failures.append(name)

    def brute():
        for causal in (0, 1):
            N, d = 6, 3
            q, k, v = pins._rand((1, 1, N, d), 1, 1.5), pins._rand((1, 1, N, d), 2, 1.5), pins._rand((1, 1, N, d), 3)
            o, lse = oracle.attention(q, k, v, causal, 0.8, lib=lib)
            o_ref, lse_ref = pins._decimal_attention(q[0, 0], k[0, 0], v[0, 0], causal, 0.8)
            np.testing.assert_allclose(o[0, 0], o_ref, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(lse[0, 0], lse_ref, rtol=1e-13, atol=1e-13)

    def rows_sum():
        for causal in (0, 1):
            N = 9
            q, k = pins._rand((1, 1, N, N), 4, 2.0), pins._rand((1, 1, N, N), 5, 2.0)
            v = np.eye(N).reshape(1, 1, N, N)
            p, _ = oracle.attention(q, k, v, causal, 0.7, lib=lib)
            assert (p >= 0).all()
            np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-13)
            if causal:
                assert np.all(p[..., np.triu(np.ones((N, N), bool), 1)] == 0)

    def zero_query():
        for causal in (0, 1):
            N, d = 8, 3
            q = np.zeros((1, 1, N, d))
            k, v = pins._rand((1, 1, N, d), 6), pins._rand((1, 1, N, d), 7)
            o, lse = oracle.attention(q, k, v, causal, 1.0, lib=lib)
            for i in range(N):
                n = i + 1 if causal else N
                np.testing.assert_allclose(lse[0, 0, i], math.log(n), atol=1e-13)
                np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n].mean(0), atol=1e-13)

    def heads():
        B, H, N, d = 1, 3, 7, 2
        q, k, v = pins._rand((B, H, N, d), 8), pins._rand((B, H, N, d), 9), pins._rand((B, H, N, d), 10)
        o, lse = oracle.attention(q, k, v, 1, 0.3, lib=lib)
        for h in range(H):
            o1, l1 = oracle.attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], 1, 0.3, lib=lib)
            np.testing.assert_array_equal(o1[0, 0], o[0, h])
            np.testing.assert_array_equal(l1[0, 0], lse[0, h])

    for name, fn in [("brute", brute), ("rows_sum", rows_sum),
                     ("zero_query", zero_query), ("heads", heads)]:
        attempt(name, fn)
    return failures


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_unmutated_oracle_passes_battery():
    assert _battery(oracle.load()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, workdir):
    old, new = MUTANTS[name]
    with open(oracle_mod._SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new)
    path_c = os.path.join(workdir, f"{name}.c")
    with open(path_c, "w") as f:
        f.write(mutated)
    lib = oracle.load(oracle.build(path_c, os.path.join(workdir, f"lib{name}.so")))
    assert _battery(lib), f"no pin caught the planted mistake {name}"
