"""The backward oracle's pins must catch plausible mistakes (no GPU).

Each case plants one mistake in a copy of oracle/bwd_oracle.py (a dropped
term, a transposed operand, a wrong scale or mask), loads the copy as a
module, and checks that the pin battery of test_bwd_oracle_pins.py fails on
it.  Mistakes are planted only in the oracle, only on the CPU.
"""
import importlib.util
import os
import sys
import types

import pytest

import oracle
import test_bwd_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "bwd_oracle.py")

MUTANTS = {
    "delta_dropped": ("ds = p * (dp - delta[:, None])", "ds = p * dp"),
    "delta_wrong_axis": ("delta = (do * o).sum(axis=1)", "delta = (do * o).sum(axis=0)"),
    "dk_untransposed": ("dk = scale * (ds.T @ q)", "dk = scale * (ds @ q)"),
    "dv_untransposed": ("dv = p.T @ do", "dv = p @ do"),
    "dq_scale_dropped": ("dq = scale * (ds @ k)", "dq = ds @ k"),
    "dk_scale_squared": ("dk = scale * (ds.T @ q)", "dk = scale * scale * (ds.T @ q)"),
    "dp_uses_k": ("dp = do @ v.T", "dp = do @ k.T"),
    "mask_transposed": ("np.tril(np.ones((N, N), dtype=bool))", "np.triu(np.ones((N, N), dtype=bool))"),
    "mask_ignored": ("if causal:\n        s = np.where", "if False:\n        s = np.where"),
    "groups_overwrite": ("dk[b, g] += gk", "dk[b, g] = gk"),
    "dq_uses_q": ("dq = scale * (ds @ k)", "dq = scale * (ds @ q)"),
    "dv_from_delta_sign": ("ds = p * (dp - delta[:, None])", "ds = p * (dp + delta[:, None])"),
}


def _load_mutant(name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    text = text.replace(old, new)
    mod = types.ModuleType(f"oracle._bwd_mutant_{name}")
    mod.__package__ = "oracle"
    exec(compile(text, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod.attention_bwd


def _battery(bwd):
    failed = []
    checks = {
        "fd": lambda: [pins.pin_finite_differences(bwd, c, H=2, Hkv=1) for c in (0, 1)],
        "single": lambda: pins.pin_single_key(bwd),
        "zero_q": lambda: pins.pin_zero_queries(bwd),
        "inv": lambda: [pins.pin_invariants(bwd, c) for c in (0, 1)],
        "groups": lambda: [pins.pin_groups_sum(bwd, c) for c in (0, 1)],
        "autograd": lambda: [pins.pin_autograd(bwd, c) for c in (0, 1)],
    }
    for name, fn in checks.items():
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            failed.append(name)
    return failed


def test_battery_passes_on_the_oracle():
    assert _battery(oracle.attention_bwd) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    bwd = _load_mutant(name, *MUTANTS[name])
    failed = _battery(bwd)
    assert failed, f"no pin caught mutant {name}"
