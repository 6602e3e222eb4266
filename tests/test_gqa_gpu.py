"""GPU parity of grouped K/V heads (fa_fwd_gqa through the binding) against
the fp64 oracle, every element: Hkv K/V heads shared by consecutive groups of
the H query heads, every dtype and head dimension, both maskings, ragged N,
and launches large enough to take the wide kernels' causal route."""
import sys

import numpy as np
import pytest
import torch

import oracle
from gates import check, widen
from io_aware_exact_05_amd import inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(dtype, d, causal, B, H, Hkv, N, seed):
    from io_aware_exact_05_amd import fa
    q = inputs.random_inputs(B, H, N, d, dtype, seed=seed)[0]
    k, v = inputs.random_inputs(B, Hkv, N, d, dtype, seed=seed + 1)[1:]
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = fa.attention(q.cuda(), k.cuda(), v.cuda(), bool(causal), scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_gqa(widen(q), widen(k), widen(v), causal, scale)
    check(o.cpu(), lse.cpu(), o_ref, lse_ref, dtype, f"{dtype} d={d} B={B} H={H} Hkv={Hkv} N={N} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("B,H,Hkv,N", [(2, 8, 2, 200), (1, 6, 1, 257), (1, 4, 4, 65)])
def test_gqa_small_every_element(dtype, d, causal, B, H, Hkv, N):
    _say(f"case gqa dtype={dtype} d={d} causal={causal} B={B} H={H} Hkv={Hkv} N={N}")
    _case(dtype, d, causal, B, H, Hkv, N, seed=H * 100 + Hkv * 10 + N)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_gqa_large_grid_causal(dtype, d):
    # more than three workgroups per CU: the wide kernel's causal route
    B, H, Hkv, N = 1, 256, 32, 400
    _say(f"case gqa large-grid dtype={dtype} d={d} H={H} Hkv={Hkv} N={N}")
    _case(dtype, d, 1, B, H, Hkv, N, seed=4242 + d)


def test_gqa_equals_repeated_kv():
    # the same launch with K/V repeated to H heads gives bit-identical results
    from io_aware_exact_05_amd import fa
    B, H, Hkv, N, d = 2, 8, 2, 300, 128
    q = inputs.random_inputs(B, H, N, d, "bf16", seed=77)[0].cuda()
    k, v = (t.cuda() for t in inputs.random_inputs(B, Hkv, N, d, "bf16", seed=78)[1:])
    idx = torch.as_tensor(oracle.gqa_kv_index(H, Hkv)).cuda()
    o1, l1 = fa.attention(q, k, v, False, 0.088)
    o2, l2 = fa.attention(q, k[:, idx].contiguous(), v[:, idx].contiguous(), False, 0.088)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_long_causal_configuration():
    # 2 x 512 causal 512-row tiles at d = 128: the long-causal configuration,
    # with four query heads per K/V head
    _say("case gqa long-causal bf16 d=128 B=2 H=256 Hkv=64 N=600")
    _case("bf16", 128, 1, 2, 256, 64, 600, seed=91)
