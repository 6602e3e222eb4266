"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Small shapes compare every element and span several tiles plus a ragged tail;
the full-size workloads run in the same launch configuration the benchmark
times and compare every element of O and the LSE with the full fp64 oracle.
Gates: |O - O_ref| <= 1e-2 + half an output ulp of O_ref, |LSE - LSE_ref| <= 1e-3.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from gates import check, widen
from io_aware_exact_05_amd import inputs

pytestmark = pytest.mark.gpu

TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _fa():
    from io_aware_exact_05_amd import fa
    return fa


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(q, k, v, causal, scale):
    fa = _fa()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse = fa.attention(qd, kd, vd, bool(causal), scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


SMALL_N = [1, 7, 64, 129, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", SMALL_N)
@pytest.mark.parametrize("causal", [0, 1])
def test_small_shapes_every_element(dtype, d, N, causal):
    B, H = (1, 2) if N >= 1000 else (2, 3)
    _say(f"case small dtype={dtype} d={d} N={N} causal={causal} B={B} H={H}")
    q, k, v = inputs.random_inputs(B, H, N, d, dtype, seed=N + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = run_gpu(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.attention(widen(q), widen(k), widen(v), causal, scale)
    st = check(o, lse, o_ref, lse_ref, dtype, f"{dtype} d={d} N={N} causal={causal}")
    if dtype == "f32":  # fp32 operands and fp32 P: far inside the gate
        assert st["o_max_abs"] < 1e-4 and st["lse_max_abs"] < 1e-4, st


# Kernel routing: d = 128 always runs fwd_pipe (256-row workgroups).  With
# causal masking at d = 64, a launch with at least two rounds of 512-row
# workgroups (one per CU) runs fwd_wide's long-causal configuration (64 rows
# per wave, ping-pong halves); otherwise, at d = 64 and 256, a launch whose
# grid exceeds one round of fwd_wide's causal slots (d = 64: 128-row
# workgroups, three per CU; d = 256: 256-row workgroups, one per CU) runs
# fwd_wide, and one that fits in a round the 8-wave 32-row fwd_mfma16.  The
# small shapes above take the fwd_mfma16 route for causal masking at d = 64
# and 256; these head counts push small, ragged causal launches onto the
# other kernels, element by element (BH = 800, N = 100 at d = 64 reaches the
# long-causal configuration, the others the 128-row one).
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("BH,N", [(800, 100), (400, 300), (260, 257)])
def test_many_heads_causal_every_element(dtype, d, BH, N):
    _say(f"case many-heads causal dtype={dtype} d={d} BH={BH} N={N}")
    q, k, v = inputs.random_inputs(1, BH, N, d, dtype, seed=BH + N)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = run_gpu(q, k, v, 1, scale)
    o_ref, lse_ref = oracle.attention(widen(q), widen(k), widen(v), 1, scale)
    check(o, lse, o_ref, lse_ref, dtype, f"{dtype} BH={BH} N={N} causal")


# Causal launches with at least two rounds of 512-row workgroups (one per
# CU, 256 CUs) take, at d = 64, the long-causal configuration of fwd_wide
# (64 rows per wave, ping-pong halves); at d = 128 the same shapes run
# fwd_pipe with many query tiles per head and diagonal tiles at every query
# tile; ragged sequence lengths, every element.
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("BH,N", [(512, 600), (256, 1030)])
def test_long_causal_configuration_every_element(dtype, d, BH, N):
    _say(f"case long-causal dtype={dtype} d={d} BH={BH} N={N}")
    q, k, v = inputs.random_inputs(1, BH, N, d, dtype, seed=BH + 7 * N + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = run_gpu(q, k, v, 1, scale)
    o_ref, lse_ref = oracle.attention(widen(q), widen(k), widen(v), 1, scale)
    check(o, lse, o_ref, lse_ref, dtype, f"{dtype} BH={BH} N={N} causal")


# At d = 128, launches with at least as many pairs of query tiles as CUs
# give each workgroup two tiles, the second one's first K/V tiles copied
# during the first one's last iterations: with causal masking tiles i and
# nq - 1 - i of one head, without it (head counts that are multiples of 16,
# key-tile counts that are multiples of the 4-stage ring) the same tile of
# two heads.  Ragged N, the middle tile of an odd count alone (N = 600),
# GQA heads.
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,H,Hkv,N,causal", [(2, 128, 128, 512, 0), (2, 128, 128, 512, 1),
                                              (1, 128, 128, 1000, 0), (1, 128, 128, 1000, 1),
                                              (1, 128, 128, 600, 1), (2, 128, 16, 512, 1),
                                              (2, 128, 16, 512, 0)])
def test_paired_query_tiles_every_element(dtype, B, H, Hkv, N, causal):
    _say(f"case paired tiles dtype={dtype} B={B} H={H} Hkv={Hkv} N={N} causal={causal}")
    d = 128
    q, _, _ = inputs.random_inputs(B, H, N, d, dtype, seed=B * H + N + causal)
    _, k, v = inputs.random_inputs(B, Hkv, N, d, dtype, seed=B * Hkv + 3 * N)
    scale = float(np.float32(1 / math.sqrt(d)))
    fa = _fa()
    o, lse = fa.attention(q.cuda(), k.cuda(), v.cuda(), bool(causal), scale)
    torch.cuda.synchronize()
    rep = H // Hkv
    kr, vr = np.repeat(widen(k), rep, axis=1), np.repeat(widen(v), rep, axis=1)
    o_ref, lse_ref = oracle.attention(widen(q), kr, vr, causal, scale)
    check(o.cpu(), lse.cpu(), o_ref, lse_ref, dtype, f"{dtype} paired B={B} H={H} N={N} causal={causal}")


# A negative scale moves into Q's sign bits, for the second query tile of a
# pair as for the first.
@pytest.mark.parametrize("causal", [0, 1])
def test_paired_query_tiles_negative_scale(causal):
    _say(f"case paired tiles negative scale causal={causal}")
    B, H, N, d = 2, 128, 512, 128
    q, k, v = inputs.random_inputs(B, H, N, d, "bf16", seed=77 + causal)
    o, lse = run_gpu(q, k, v, causal, -0.3)
    o_ref, lse_ref = oracle.attention(widen(q), widen(k), widen(v), causal, -0.3)
    check(o, lse, o_ref, lse_ref, "bf16", f"paired negative scale causal={causal}")


FULL = [w for w in inputs.WORKLOADS if w.dtype != "e4m3"]


@pytest.mark.parametrize("w", FULL, ids=lambda w: f"{w.name}.{w.case_id}")
def test_workload_full_size_every_element(w):
    """Every element of O and the LSE of each full-size workload against the
    full fp64 oracle (the result is exact up to rounding, "FlashAttention
    (HI)", online-softmax section, so one gate holds for every element)."""
    _say(f"case workload {w.label()}")
    q, k, v = inputs.workload_inputs(w)
    o, lse = run_gpu(q, k, v, w.causal, w.scale)
    o_ref, lse_ref = oracle.attention(widen(q), widen(k), widen(v), w.causal, w.scale)
    st = check(o, lse, o_ref, lse_ref, w.dtype, w.label())
    _say(f"  {w.label()}: {st}")


# ----------------------------- edge cases ---------------------------------

@pytest.mark.parametrize("scale", [-0.3, 0.0, 1.5])
@pytest.mark.parametrize("causal", [0, 1])
def test_unusual_scales(scale, causal):
    _say(f"case scale={scale} causal={causal}")
    q, k, v = inputs.random_inputs(1, 2, 300, 128, "bf16", seed=5)
    o, lse = run_gpu(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.attention(widen(q), widen(k), widen(v), causal, scale)
    check(o, lse, o_ref, lse_ref, "bf16", f"scale={scale}")


@pytest.mark.parametrize("BH", [(1, 8), (2, 8), (1, 9), (3, 5)])
def test_head_counts_and_block_mapping(BH):
    B, H = BH
    _say(f"case B={B} H={H}")
    for causal in (0, 1):
        q, k, v = inputs.random_inputs(B, H, 260, 64, "f16", seed=B * 10 + H)
        o, lse = run_gpu(q, k, v, causal, 0.125)
        o_ref, lse_ref = oracle.attention(widen(q), widen(k), widen(v), causal, 0.125)
        check(o, lse, o_ref, lse_ref, "f16", f"B={B} H={H} causal={causal}")


@pytest.mark.parametrize("causal", [0, 1])
def test_constant_v_gives_constant_output(causal):
    _say(f"case constant V causal={causal}")
    q, k, _ = inputs.random_inputs(2, 2, 200, 128, "bf16", seed=7)
    c = torch.randn(2, 2, 1, 128).to(torch.bfloat16)
    v = c.expand(2, 2, 200, 128).contiguous()
    o, _ = run_gpu(q, k, v, causal, 0.09)
    np.testing.assert_allclose(widen(o), np.broadcast_to(widen(c), o.shape), atol=1e-2, rtol=4e-3)


@pytest.mark.parametrize("causal", [0, 1])
def test_identity_v_rows_of_p_sum_to_one(causal):
    _say(f"case identity V causal={causal}")
    N = d = 64
    q, k, _ = inputs.random_inputs(1, 1, N, d, "f16", seed=9)
    v = torch.eye(N, dtype=torch.float16).reshape(1, 1, N, d)
    p, _ = run_gpu(q, k, v, causal, 0.3)
    p = widen(p)[0, 0]
    assert (p >= 0).all()
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-2)
    if causal:
        assert (p[np.triu(np.ones((N, N), bool), 1)] == 0).all()


def test_deterministic_bitwise():
    _say("case determinism")
    q, k, v = inputs.random_inputs(2, 8, 700, 128, "bf16", seed=11)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    fa = _fa()
    outs = []
    for causal in (0, 1):
        ref = None
        for _ in range(3):
            o, lse = fa.attention(qd, kd, vd, bool(causal), 0.088)
            torch.cuda.synchronize()
            if ref is None:
                ref = (o.clone(), lse.clone())
            else:
                assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1])


@pytest.mark.parametrize("dtype,B,H,N", [("bf16", 1, 3, 333), ("f32", 1, 3, 333), ("bf16", 1, 128, 1000)])
def test_every_output_written_and_no_out_of_bounds_writes(dtype, B, H, N):
    _say(f"case poison/canary {dtype} B={B} H={H} N={N}")
    d = 128
    q, k, v = inputs.random_inputs(B, H, N, d, dtype, seed=13)
    fa = _fa()
    n, guard = B * H * N * d, 4096
    obuf = torch.full((n + 2 * guard,), float("nan"), dtype=TORCH[dtype], device="cuda")
    lbuf = torch.full((B * H * N + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
    obuf[:guard] = 7.0; obuf[-guard:] = 7.0
    lbuf[:guard] = 7.0; lbuf[-guard:] = 7.0
    o = obuf[guard:guard + n].view(B, H, N, d)
    lse = lbuf[guard:guard + B * H * N].view(B, H, N)
    for causal in (0, 1):
        fa.fa_fwd(q.cuda(), k.cuda(), v.cuda(), o, lse, bool(causal), 0.088)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        assert (obuf[:guard] == 7).all() and (obuf[-guard:] == 7).all()
        assert (lbuf[:guard] == 7).all() and (lbuf[-guard:] == 7).all()


def test_status_errors_on_device_tensors():
    _say("case error statuses")
    fa = _fa()
    q = torch.zeros(1, 1, 16, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.attention(q, q, q)
    assert e.value.status == -4
    q = torch.zeros(1, 1, 16, 64, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(1, 1, 16, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd(q, q, q, q, lse, False, 0.1)  # o aliases the inputs
    assert e.value.status == -7
