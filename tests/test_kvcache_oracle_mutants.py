"""The KV-cache oracle's pins must catch plausible mistakes (no GPU): each
case plants one mistake in a copy of oracle/kvcache_oracle.py and checks that
the pins of test_kvcache_oracle_pins.py fail on it."""
import os
import types

import pytest

import oracle
import test_kvcache_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kvcache_oracle.py")

MUTANTS = {
    "top_left_mask": ("<= (Nkv - Nq + np.arange(Nq))", "<= (np.arange(Nq))"),
    "mask_off_by_one": ("<= (Nkv - Nq + np.arange(Nq))", "< (Nkv - Nq + np.arange(Nq))"),
    "mask_ignored": ("if causal:\n                s = np.where", "if False:\n                s = np.where"),
    "lse_without_max": ("lse[b, h] = (m + np.log(l))[:, 0]", "lse[b, h] = np.log(l)[:, 0]"),
    "head_map_modulo": ("g = kv_of[h]", "g = h % Hkv"),
    "scale_dropped": ("s = scale * (q[b, h] @ k[b, g].T)", "s = q[b, h] @ k[b, g].T"),
    "unnormalised": ("o[b, h] = (e / l) @ v[b, g]", "o[b, h] = e @ v[b, g]"),
}


def _mutant(old, new):
    text = open(SRC).read()
    assert text.count(old) == 1
    mod = types.ModuleType("oracle._kv_mutant")
    mod.__package__ = "oracle"
    exec(compile(text.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    return mod.attention_kvcache


PINS = [
    lambda: [pins.test_equal_lengths_match_the_c_oracle(c) for c in (0, 1)],
    lambda: [pins.test_decoded_rows_are_the_last_rows_of_a_causal_prefill(n) for n in (1, 3, 16)],
    pins.test_single_query_sees_the_whole_cache_either_way,
    pins.test_identical_keys_average_the_values,
    lambda: [pins.test_decimal_brute_force(c) for c in (0, 1)],
    lambda: [pins.test_split_merge_identity(c) for c in (1, 17, 39)],
    pins.test_shared_heads_match_the_grouped_oracle,
]


def _failures(fn, monkeypatch):
    monkeypatch.setattr(oracle, "attention_kvcache", fn)
    failed = 0
    for p in PINS:
        try:
            p()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    return failed


def test_pins_pass_on_the_oracle(monkeypatch):
    assert _failures(oracle.attention_kvcache, monkeypatch) == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    assert _failures(_mutant(*MUTANTS[name]), monkeypatch) > 0, name
