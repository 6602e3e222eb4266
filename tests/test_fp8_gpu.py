"""GPU tests of the fp8 path through the C ABI.

Quantiser: e4m3 codes and descales against the fp32-precision oracle — bit
for bit without rotation; within one code step (and descales within 2e-6)
with the randomised Hadamard rotation, whose fp32 butterflies round
differently from the oracle's fp64 matrix product.
Attention, end to end: fp8 output against the fp64 oracle run on the
UNQUANTISED fp32 inputs, gated on the whole-tensor relative RMSE <= 5e-2.
Attention kernel alone: the oracle runs on exactly the values the codes
stand for, and every output element must lie within a bound derived from
the kernel's arithmetic (see _fp8_kernel_bounds).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from gates import widen
from io_aware_exact_05_amd import inputs
from oracle import quant_oracle as qo

pytestmark = pytest.mark.gpu

REL_RMSE_GATE = 5e-2


def _fa():
    from io_aware_exact_05_amd import fa
    return fa


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _ordinal(codes):
    c = np.asarray(codes, np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def _rel_rmse(o, ref):
    o, ref = np.asarray(o, np.float64), np.asarray(ref, np.float64)
    return float(np.linalg.norm(o - ref) / np.linalg.norm(ref))


def _fp32_inputs(B, H, N, d, seed, outliers="entries_x10"):
    return inputs.random_inputs(B, H, N, d, "e4m3", seed=seed, outliers=outliers)


QSHAPES = [(1, 2, 300, 64), (2, 1, 128, 128), (1, 1, 1000, 256), (1, 3, 129, 128), (1, 1, 1, 128)]


@pytest.mark.parametrize("shape", QSHAPES, ids=lambda s: "x".join(map(str, s)))
def test_quantizer_bitwise_without_rotation(shape):
    _say(f"case quantize no-rotation {shape}")
    fa = _fa()
    x, _, _ = _fp32_inputs(*shape, seed=sum(shape))
    if shape[2] >= 256:
        x[:, :, 128:256] = 0.0  # an all-zero block
    x8, desc = fa.quantize_e4m3(x.cuda(), rotate=False)
    torch.cuda.synchronize()
    codes_ref, desc_ref = qo.quantize_blocks(x.numpy(), 128)
    np.testing.assert_array_equal(desc.cpu().numpy(), desc_ref)
    np.testing.assert_array_equal(x8.cpu().numpy(), codes_ref)


@pytest.mark.parametrize("shape", QSHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("with_signs", [True, False])
def test_quantizer_with_rotation_within_one_code(shape, with_signs):
    _say(f"case quantize rotation {shape} signs={with_signs}")
    fa = _fa()
    d = shape[-1]
    x, _, _ = _fp32_inputs(*shape, seed=3 * sum(shape))
    signs = inputs.rotation_signs(d, seed=1) if with_signs else None
    x8, desc = fa.quantize_e4m3(x.cuda(), rotate=True,
                                signs=signs.cuda() if signs is not None else None)
    torch.cuda.synchronize()
    codes_ref, desc_ref = qo.quantize_blocks(x.numpy(), 128,
                                             signs.numpy() if signs is not None else None, True)
    np.testing.assert_allclose(desc.cpu().numpy(), desc_ref, rtol=2e-6, atol=0)
    diff = np.abs(_ordinal(x8.cpu().numpy()) - _ordinal(codes_ref))
    assert diff.max() <= 1, diff.max()
    assert (diff > 0).mean() < 0.01


# Error terms of the fp8 kernel on exactly-representable inputs:
#  * P is rounded to e4m3 for the second product: relative error <= 2^-4 for
#    normal codes; below 2^-6 (subnormal codes) an absolute error <= 2^-10 in
#    units where P <= 2^8 at the running max, i.e. <= 2^-16 times the row max
#    of exp(s - max s) (the running max sits at most 2 binades below the true
#    one, which only shrinks this);
#  * the fp8 MFMA's dot products are not exact in fp32: measured on gfx950,
#    a 64-term product differs from the exact sum by at most 2^-11.3 of its
#    largest term and 2^-11.9 of the sum of its term magnitudes; 2^-10 of the
#    sum of magnitudes is used as the bound, for the scores and for P V;
#  * bf16 output rounding: 2^-9 relative.
# Statistically, RNE to 3 mantissa bits of log-uniform values has a relative
# RMS error of 2^-4 / sqrt(3) * sqrt(3 / (8 ln 2)) = 0.0265, which bounds the
# whole-tensor relative RMSE of O (errors of independent keys average).
KERNEL_REL_RMSE = 3e-2
SCORE_ERR = 2.0 ** -10


def _fp8_kernel_bounds(Qd, Kd, Vd, causal, scale, o_ref, lse_ref):
    """Per-element bound on |O - O_ref| and per-row bound on |LSE - LSE_ref|."""
    sabs = np.abs(Qd) @ np.swapaxes(np.abs(Kd), 2, 3)
    if causal:
        N = Qd.shape[2]
        sabs = np.where(np.tril(np.ones((N, N), bool))[None, None], sabs, 0.0)
    ds = abs(scale) * SCORE_ERR * sabs.max(axis=3)          # score error per row
    lse_tol = ds + 1e-5 * (1.0 + np.abs(lse_ref))
    att_abs, _ = oracle.attention(Qd, Kd, np.abs(Vd), causal, scale)
    va = np.abs(Vd)
    vsum = np.cumsum(va, axis=2) if causal else np.broadcast_to(va.sum(axis=2, keepdims=True), va.shape)
    grow = np.expm1(2.0 * ds)[..., None]                    # P and l both move by exp(+-ds)
    o_tol = ((2.0 ** -4) * (1.0 + grow) + grow + SCORE_ERR) * att_abs + 2.0 ** -16 * vsum \
        + 2.0 ** -8 * np.abs(o_ref) + 1e-6
    return o_tol, lse_tol


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [1, 7, 129, 300, 1000])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("rotate", [True, False])
def test_fp8_kernel_on_oracle_quantised_inputs(d, N, causal, rotate):
    """The attention kernel alone: Q, K, V are quantised by the oracle (with
    the rotation when asked), the kernel gets those codes and descales, and
    the fp64 oracle runs on exactly the values the codes stand for."""
    _say(f"case fp8 kernel d={d} N={N} causal={causal} rotate={rotate}")
    fa = _fa()
    B, H = 1, 2
    q, k, v = _fp32_inputs(B, H, N, d, seed=N + 11)
    scale = float(np.float32(1 / math.sqrt(d)))
    signs = inputs.rotation_signs(d, seed=2).numpy() if rotate else None
    cq, dq = qo.quantize_blocks(q.numpy(), 128, signs, rotate)
    ck, dk = qo.quantize_blocks(k.numpy(), 128, signs, rotate)
    cv, dv = qo.quantize_blocks(v.numpy(), 128)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), device="cuda")
    fa.fa_fwd_fp8(dev(cq), dev(ck), dev(cv), dev(dq), dev(dk), dev(dv), o, lse, bool(causal), scale)
    torch.cuda.synchronize()
    Qd, Kd, Vd = (qo.dequantize_blocks(c, ds) for c, ds in ((cq, dq), (ck, dk), (cv, dv)))
    o_ref, lse_ref = oracle.attention(Qd, Kd, Vd, causal, scale)
    o_np, lse_np = widen(o.cpu()), widen(lse.cpu())
    assert np.isfinite(o_np).all() and np.isfinite(lse_np).all()
    o_tol, lse_tol = _fp8_kernel_bounds(Qd, Kd, Vd, causal, scale, o_ref, lse_ref)
    err = _rel_rmse(o_np, o_ref)
    ro = float((np.abs(o_np - o_ref) / o_tol).max())
    rl = float((np.abs(lse_np - lse_ref) / lse_tol).max())
    _say(f"  rel-RMSE {err:.5f}  worst |dO|/bound {ro:.3f}  worst |dLSE|/bound {rl:.3f}")
    assert err <= KERNEL_REL_RMSE
    assert ro <= 1.0 and rl <= 1.0


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [300, 1000])
@pytest.mark.parametrize("causal", [0, 1])
def test_fp8_kernel_descales_not_powers_of_two(d, N, causal):
    """The kernel with caller-supplied descales that are not powers of two
    (this library's quantiser only writes powers of two).  A V descale
    2^e f with f in (1/2, 1) puts log2 f into the exponent of P~ and 1/f
    into the row sum; Q and K descales enter the score scale.  Codes come
    from the oracle's quantiser, every descale is then replaced by a random
    value in [0.002, 0.05), and the fp64 oracle runs on the values the codes
    and those descales stand for, under the kernel-alone bounds."""
    _say(f"case fp8 kernel arbitrary descales d={d} N={N} causal={causal}")
    fa = _fa()
    B, H = 1, 2
    q, k, v = _fp32_inputs(B, H, N, d, seed=N + 5 * d + causal)
    scale = float(np.float32(1 / math.sqrt(d)))
    rng = np.random.default_rng(N + d)
    codes, descs = [], []
    for x in (q, k, v):
        c, ds = qo.quantize_blocks(x.numpy(), 128)
        codes.append(c)
        descs.append(rng.uniform(0.002, 0.05, ds.shape).astype(np.float32))
    mant = np.frexp(descs[2])[0]
    assert (mant != 0.5).all()  # no power of two among the V descales
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), device="cuda")
    fa.fa_fwd_fp8(*(dev(c) for c in codes), *(dev(ds) for ds in descs), o, lse, bool(causal), scale)
    torch.cuda.synchronize()
    Qd, Kd, Vd = (qo.dequantize_blocks(c, ds) for c, ds in zip(codes, descs))
    o_ref, lse_ref = oracle.attention(Qd, Kd, Vd, causal, scale)
    o_np, lse_np = widen(o.cpu()), widen(lse.cpu())
    assert np.isfinite(o_np).all() and np.isfinite(lse_np).all()
    o_tol, lse_tol = _fp8_kernel_bounds(Qd, Kd, Vd, causal, scale, o_ref, lse_ref)
    err = _rel_rmse(o_np, o_ref)
    ro = float((np.abs(o_np - o_ref) / o_tol).max())
    rl = float((np.abs(lse_np - lse_ref) / lse_tol).max())
    _say(f"  rel-RMSE {err:.5f}  worst |dO|/bound {ro:.3f}  worst |dLSE|/bound {rl:.3f}")
    assert err <= KERNEL_REL_RMSE
    assert ro <= 1.0 and rl <= 1.0


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("scale", [-0.3, 0.0])
def test_fp8_kernel_negative_and_zero_scale(d, causal, scale):
    """A negative softmax scale reaches the kernel as Q codes with flipped
    sign bits and |scale|; a zero scale makes every visible key's weight
    equal (O the mean of the visible V rows, LSE the log of their count).
    Oracle-quantised inputs, N = 300 (a ragged third block), kernel-alone
    bounds."""
    _say(f"case fp8 kernel scale={scale} d={d} causal={causal}")
    fa = _fa()
    B, H, N = 1, 2, 300
    q, k, v = _fp32_inputs(B, H, N, d, seed=17 * d + causal)
    cq, dq = qo.quantize_blocks(q.numpy(), 128)
    ck, dk = qo.quantize_blocks(k.numpy(), 128)
    cv, dv = qo.quantize_blocks(v.numpy(), 128)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), device="cuda")
    fa.fa_fwd_fp8(dev(cq), dev(ck), dev(cv), dev(dq), dev(dk), dev(dv), o, lse, bool(causal), scale)
    torch.cuda.synchronize()
    Qd, Kd, Vd = (qo.dequantize_blocks(c, ds) for c, ds in ((cq, dq), (ck, dk), (cv, dv)))
    o_ref, lse_ref = oracle.attention(Qd, Kd, Vd, causal, scale)
    o_np, lse_np = widen(o.cpu()), widen(lse.cpu())
    assert np.isfinite(o_np).all() and np.isfinite(lse_np).all()
    o_tol, lse_tol = _fp8_kernel_bounds(Qd, Kd, Vd, causal, scale, o_ref, lse_ref)
    ro = float((np.abs(o_np - o_ref) / o_tol).max())
    rl = float((np.abs(lse_np - lse_ref) / lse_tol).max())
    _say(f"  worst |dO|/bound {ro:.3f}  worst |dLSE|/bound {rl:.3f}")
    assert ro <= 1.0 and rl <= 1.0


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [0, 1])
def test_fp8_attention_exactly_representable_inputs(d, causal):
    """Values in {0, +-1/2, +-1} with one 8 per block and column are quantised
    without error (the descale 2^-5 maps them onto the e4m3 codes of 0, 16,
    32 and 256), so the end-to-end result obeys the kernel-only bounds."""
    _say(f"case fp8 exact inputs d={d} causal={causal}")
    fa = _fa()
    B, H, N = 1, 2, 384
    rng = np.random.default_rng(5)
    vals = np.array([-1.0, -0.5, 0.0, 0.5, 1.0], np.float32)
    qkv = []
    for _ in range(3):
        x = rng.choice(vals, (B, H, N, d)).astype(np.float32)
        x[:, :, ::128, :] = 8.0
        qkv.append(torch.from_numpy(x))
    q, k, v = qkv
    scale = 0.125
    o, lse = fa.attention_fp8(q.cuda(), k.cuda(), v.cuda(), bool(causal), scale, False)
    torch.cuda.synchronize()
    for x in (q, k, v):  # the quantiser really is lossless here
        c, ds = qo.quantize_blocks(x.numpy(), 128)
        np.testing.assert_array_equal(qo.dequantize_blocks(c, ds), x.numpy())
    Qd, Kd, Vd = widen(q), widen(k), widen(v)
    o_ref, lse_ref = oracle.attention(Qd, Kd, Vd, causal, scale)
    o_np, lse_np = widen(o.cpu()), widen(lse.cpu())
    o_tol, lse_tol = _fp8_kernel_bounds(Qd, Kd, Vd, causal, scale, o_ref, lse_ref)
    err = _rel_rmse(o_np, o_ref)
    ro = float((np.abs(o_np - o_ref) / o_tol).max())
    rl = float((np.abs(lse_np - lse_ref) / lse_tol).max())
    _say(f"  rel-RMSE {err:.5f}  worst |dO|/bound {ro:.3f}  worst |dLSE|/bound {rl:.3f}")
    assert err <= KERNEL_REL_RMSE
    assert ro <= 1.0 and rl <= 1.0


@pytest.mark.parametrize("case", [0, 1, 2, 3])
def test_fp8_workload_rotation_and_without(case):
    """Whole-tensor relative RMSE of the fp8 workload and its variants
    against the fp64 oracle on the unquantised fp32 inputs, with and without
    the rotation of Q and K.  Case 0 is the fp8 configuration (d = 128,
    non-causal); 1-3 its d = 64, d = 256 and causal variants.  The 5e-2 gate
    holds for cases 0, 2 and 3; at d = 64 the rotation spreads an outlier
    over only 64 columns and the end-to-end error stays above it (reported,
    not gated; the kernel arithmetic of that variant is gated element by
    element in test_fp8_kernel_on_oracle_quantised_inputs)."""
    w = inputs.workload(5, case)
    _say(f"case fp8 workload {w.label()}")
    fa = _fa()
    q, k, v = inputs.workload_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    signs = inputs.rotation_signs(w.d, seed=0).cuda()
    o_ref, lse_ref = oracle.attention(widen(q), widen(k), widen(v), w.causal, w.scale)
    errs = {}
    for rot in (True, False):
        o, lse = fa.attention_fp8(qd, kd, vd, bool(w.causal), w.scale, rot, signs if rot else None)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        errs[rot] = (_rel_rmse(widen(o.cpu()), o_ref), float(np.abs(widen(lse.cpu()) - lse_ref).max()))
    _say(f"  rel-RMSE with rotation {errs[True][0]:.4f} (max|dLSE| {errs[True][1]:.4f}); "
         f"without {errs[False][0]:.4f} (max|dLSE| {errs[False][1]:.4f}); "
         f"ratio {errs[False][0] / errs[True][0]:.2f}")
    assert errs[True][0] <= errs[False][0]  # the rotation never makes it worse
    if w.d != 64:
        assert errs[True][0] <= REL_RMSE_GATE


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp8_mfma_dot_product_error(d):
    """The premise of the kernel-alone fp8 bound: a dot product of e4m3
    values on the scaled fp8 MFMA lies within 2^-10 of the sum of the terms'
    magnitudes of the exact value.  With one key per head the kernel's only
    score is S = q . k (descales 1), P = 1, l = 1, so LSE = scale S up to
    three fp32 roundings; 2048 heads of random finite codes, and 2048 of
    codes of quantised normal data, through the C ABI."""
    fa = _fa()
    rng = np.random.default_rng(9000 + d)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    for kind in ("uniform codes", "quantised normals"):
        BH = 2048
        if kind == "uniform codes":
            q8 = rng.choice(finite, size=(1, BH, 1, d))
            k8 = rng.choice(finite, size=(1, BH, 1, d))
        else:
            q8 = qo.e4m3_encode(rng.standard_normal((1, BH, 1, d)) * 64.0)
            k8 = qo.e4m3_encode(rng.standard_normal((1, BH, 1, d)) * 64.0)
        terms = qo.e4m3_decode(q8).astype(np.float64) * qo.e4m3_decode(k8).astype(np.float64)
        exact = terms.sum(-1)[..., 0]
        mag = np.abs(terms).sum(-1)[..., 0]
        scale = 2.0 ** -12
        one = torch.ones((1, BH, 1), dtype=torch.float32, device="cuda")
        o = torch.empty((1, BH, 1, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((1, BH, 1), dtype=torch.float32, device="cuda")
        tq = torch.from_numpy(np.ascontiguousarray(q8)).cuda()
        tk = torch.from_numpy(np.ascontiguousarray(k8)).cuda()
        tv = torch.zeros_like(tq)
        fa.fa_fwd_fp8(tq, tk, tv, one, one, one, o, lse, False, scale)
        torch.cuda.synchronize()
        s_gpu = widen(lse.cpu())[..., 0] / scale
        err = np.abs(s_gpu - exact)
        bound = 2.0 ** -10 * mag + 4 * 2.0 ** -24 * np.abs(exact)
        worst = float((err / np.maximum(bound, 1e-300)).max())
        _say(f"  d={d} {kind}: max |S - exact| / (sum|terms|) = {float((err / np.maximum(mag, 1e-300)).max()):.3e}"
             f"  (2^{np.log2(max(float((err / np.maximum(mag, 1e-300)).max()), 1e-30)):.1f}); worst/bound {worst:.3f}")
        assert np.isfinite(s_gpu).all()
        assert (err <= bound).all(), worst


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp8_deterministic_and_fully_written(d):
    _say(f"case fp8 determinism/poison d={d}")
    fa = _fa()
    B, H, N = 1, 3, 333
    q, k, v = _fp32_inputs(B, H, N, d, seed=77)
    q8, qd = fa.quantize_e4m3(q.cuda(), True)
    k8, kd = fa.quantize_e4m3(k.cuda(), True)
    v8, vd = fa.quantize_e4m3(v.cuda(), False)
    ref = None
    for _ in range(3):
        o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, H, N), float("nan"), device="cuda")
        fa.fa_fwd_fp8(q8, k8, v8, qd, kd, vd, o, lse, False, 0.088)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        if ref is None:
            ref = (o.clone(), lse.clone())
        else:
            assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1])
