"""Pins for the fp8 quantisation oracle (no GPU).

The e4m3fn codec is pinned to the OCP format definition (spot values, every
finite code round-trips, ties go to the even mantissa, saturation) and to an
independent library encoder (torch.float8_e4m3fn) on in-range values; the
randomised Hadamard rotation to its defining properties (H H^T = d I,
orthogonality, Q K^T invariance, a butterfly transform written here); the
block quantiser to amax/descale identities and its error bound.
"""
import math

import numpy as np
import pytest
import torch

from oracle import quant_oracle as qo


def test_decode_spot_values_from_the_format_definition():
    v = qo.e4m3_decode([0x00, 0x80, 0x38, 0xB8, 0x7E, 0xFE, 0x01, 0x08, 0x07, 0x40, 0x30, 0x7F])
    np.testing.assert_array_equal(v[:11], [0.0, -0.0, 1.0, -1.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -6,
                                            7 * 2.0 ** -9, 2.0, 0.5])
    assert math.isnan(v[11])


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    np.testing.assert_array_equal(qo.e4m3_encode(qo.e4m3_decode(codes)), codes)


def test_ties_round_to_even_and_neighbours_to_nearest():
    pos = np.array([c for c in range(0x7E)], np.uint8)  # 0 .. 0x7D, the next code exists
    lo, hi = qo.e4m3_decode(pos), qo.e4m3_decode(pos + 1)
    mid = (lo + hi) / 2
    got = qo.e4m3_encode(mid)
    want = np.where(pos % 2 == 0, pos, pos + 1)  # even mantissa <=> even code here
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(qo.e4m3_encode(np.nextafter(mid, 0)), pos)
    np.testing.assert_array_equal(qo.e4m3_encode(np.nextafter(mid, 1e9)), pos + 1)


def test_saturation():
    x = np.array([448.0, 449.0, 463.9, 464.0, 465.0, 1e6, 3e38, -500.0, np.inf, -np.inf])
    np.testing.assert_array_equal(qo.e4m3_encode(x), [0x7E] * 7 + [0xFE, 0x7E, 0xFE])


def test_matches_torch_float8_e4m3fn_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * 40,
                        rng.standard_normal(50000) * 1e-2,
                        rng.uniform(-448, 448, 50000)]).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(qo.e4m3_encode(x), ref)


def _fwht(x):
    """Fast Walsh-Hadamard transform of the last axis by butterflies (natural order)."""
    y = np.array(x, dtype=np.float64)
    n = y.shape[-1]
    h = 1
    while h < n:
        y = y.reshape(*y.shape[:-1], n // (2 * h), 2, h)
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :], y[..., 1, :] = a + b, a - b
        y = y.reshape(*y.shape[:-3], n)
        h *= 2
    return y


@pytest.mark.parametrize("d", [64, 128, 256])
def test_hadamard_and_rotation_properties(d):
    h = qo.hadamard(d)
    np.testing.assert_array_equal(h @ h.T, d * np.eye(d))
    rng = np.random.default_rng(d)
    signs = rng.choice([-1.0, 1.0], d)
    m = qo.rotation(d, signs)
    np.testing.assert_allclose(m @ m.T, np.eye(d), atol=1e-13)
    x = rng.standard_normal((5, d))
    np.testing.assert_allclose(x @ h, _fwht(x), atol=1e-12)
    q, k = rng.standard_normal((7, d)), rng.standard_normal((9, d))
    np.testing.assert_allclose((q @ m) @ (k @ m).T, q @ k.T, atol=1e-12)


def test_pow2_descale_definition():
    amax = np.array([448.0, 448.0001, 224.0, 1.0, 3.5, 7.0, 1e-3, 0.0, 896.0, 895.9])
    ds = qo.pow2_descale(amax)
    np.testing.assert_array_equal(ds, [1.0, 2.0, 0.5, 2.0 ** -8, 2.0 ** -7, 2.0 ** -6, 2.0 ** -18,
                                       1.0, 2.0, 2.0])
    nz = amax > 0
    assert (amax[nz] <= 448 * ds[nz]).all() and (amax[nz] > 224 * ds[nz]).all()


def test_block_quantiser_identities():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 2, 300, 64)).astype(np.float32)
    x[0, 1, 128:256] = 0.0  # an all-zero block
    codes, desc = qo.quantize_blocks(x, 128)
    assert desc.shape == (1, 2, 3)
    assert desc[0, 1, 1] == 1.0 and (codes[0, 1, 128:256] & 0x7F == 0).all()
    for h in range(2):
        for b in range(3):
            blk = x[0, h, b * 128:(b + 1) * 128]
            if np.abs(blk).max() == 0:
                continue
            amax = float(np.abs(blk).max())
            ds = float(desc[0, h, b])
            assert math.log2(ds) == round(math.log2(ds))          # a power of two
            assert amax <= 448 * ds and amax > 224 * ds             # the smallest such
            # codes are the single e4m3 rounding of x / descale
            np.testing.assert_array_equal(codes[0, h, b * 128:(b + 1) * 128],
                                          qo.e4m3_encode(blk.astype(np.float64) / ds))
    # dequantised values are within half a code step (relative 1/16) or the subnormal step
    deq = qo.dequantize_blocks(codes, desc)
    scale = np.repeat(desc, 128, axis=2)[:, :, :300, None]
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) / 16.0, 2.0 ** -10 * scale) * 1.0001
    assert (err <= bound).all()


def test_rotated_quantisation_inverts_back():
    """Dequantising rotated codes and applying M^T recovers x within the fp8
    error bound (M orthogonal): |x - deq(x M) M^T| stays at e4m3's relative
    step (2^-4) times the block scale."""
    rng = np.random.default_rng(2)
    shape = (1, 1, 256, 128)
    x = rng.standard_normal(shape)
    x[rng.random(shape) < 0.001] *= 10
    x = x.astype(np.float32)
    signs = rng.choice([-1.0, 1.0], 128)
    codes, desc = qo.quantize_blocks(x, 128, signs, True)
    back = qo.dequantize_blocks(codes, desc) @ qo.rotation(128, signs).T
    rel = np.linalg.norm(back - x) / np.linalg.norm(x)
    assert rel < 2.0 ** -4, rel
