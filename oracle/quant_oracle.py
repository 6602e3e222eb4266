"""fp8 block-quantisation oracle — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU leg may use it;
the GPU library never does.  Written from the pages' description of the fp8
path ("FlashAttention-3 (BN)" / "FlashAttention-3 (FA)", section on low
precision and reducing quantisation error) plus the OCP 8-bit floating-point
format definition:

* e4m3fn codes: sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no
  infinities, S.1111.111 is NaN, so the largest finite magnitude is
  1.75 * 2^8 = 448; exponent field 0 holds subnormals m/8 * 2^-6.
* Incoherent processing: before quantising, Q and K are multiplied by a
  random orthogonal matrix.  The plainest reading used here: the randomised
  Hadamard matrix M = H_d diag(sigma) / sqrt(d) (H_d the Sylvester Hadamard
  matrix of order d, sigma in {+1,-1}^d), applied as x <- x M to every row.
  M M^T = I, so (Q M)(K M)^T = Q K^T.
* Block quantisation (reading of the fp32 per-128-row scale): a block is 128
  consecutive sequence rows of one (b, h) with all d columns; amax is the
  block's largest magnitude; the descale is the smallest power of two
  2^e with amax <= 448 * 2^e (an fp32 value), and codes =
  e4m3_rne_saturate(x * 2^-e).  Scaling by a power of two is exact, so the
  code is the single e4m3 rounding of x / descale, the block's largest
  magnitude lands in [224, 448], and every later use of the scale (in fp32
  arithmetic or as an MFMA power-of-two block scale) is exact.  An all-zero
  block gets descale 1 and zero codes.

Without rotation every step is exact up to the one e4m3 rounding, so codes
and descales are bit-identical on any correct implementation.  The rotation
is computed here in fp64 from the matrix definition and rounded once to
fp32, so rotated codes may differ from a GPU's by one code step where its
fp32 butterflies round differently.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """uint8 e4m3fn codes -> float64 values (NaN codes -> nan)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def e4m3_encode(x) -> np.ndarray:
    """float -> uint8 e4m3fn code, round to nearest even, saturating at +-448.

    Each value is rounded on the grid of its binade (spacing 2^(e-3) for a
    normal value 2^e <= |x| < 2^(e+1), spacing 2^-9 below 2^-6); ties go to
    the even mantissa; magnitudes that round above 448 become 448.  Exact in
    fp64 for every fp32 input.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x)
    a = np.abs(x)
    out = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: multiples of 2^-9
    q = np.rint(a * 2.0 ** 9)  # numpy rint: round half to even
    out = np.where(sub, q.astype(np.int64), out)  # q == 8 is the code of 2^-6 as well
    # normal range
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.floor(np.log2(np.where(sub, 1.0, a)))
    frac = np.where(sub, 1.0, a) / np.exp2(e)  # in [1, 2)
    mq = np.rint((frac - 1.0) * 8.0)
    e = np.where(mq == 8, e + 1, e)
    mq = np.where(mq == 8, 0, mq)
    norm_code = ((e + 7) * 8 + mq).astype(np.int64)
    norm_code = np.where((e > 8) | ((e == 8) & (mq > 6)), 0x7E, norm_code)
    out = np.where(sub, out, norm_code)
    out = np.where(np.isnan(x), 0x7F, out)
    return (out | np.where(sign, 0x80, 0)).astype(np.uint8)


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two), entries +-1."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation(d: int, signs=None) -> np.ndarray:
    """M = H_d diag(signs) / sqrt(d) in fp64 (signs None = all +1)."""
    s = np.ones(d) if signs is None else np.asarray(signs, dtype=np.float64)
    return hadamard(d) * s[None, :] / math.sqrt(d)


def rotate(x, signs=None) -> np.ndarray:
    """x [..., d] -> x M, computed in fp64 and rounded once to fp32."""
    x = np.asarray(x, dtype=np.float64)
    return (x @ rotation(x.shape[-1], signs)).astype(np.float32)


def pow2_descale(amax) -> np.ndarray:
    """Smallest power of two 2^e with amax <= 448 * 2^e (1 where amax == 0)."""
    a = np.asarray(amax, dtype=np.float64)
    e = np.ceil(np.log2(np.where(a > 0, a, 1.0) / E4M3_MAX))
    # guard the floating-point log2 at exact powers: enforce the defining inequalities
    e = np.where(a > E4M3_MAX * np.exp2(e), e + 1, e)
    e = np.where(a <= E4M3_MAX * np.exp2(e - 1), e - 1, e)
    return np.where(a > 0, np.exp2(e), 1.0).astype(np.float32)


def quantize_blocks(x, block_rows: int = 128, rotate_signs=None, do_rotate: bool = False):
    """x fp32 [B, H, N, d] -> (codes uint8 [B,H,N,d], descale fp32 [B,H,ceil(N/block_rows)])."""
    x = np.asarray(x, dtype=np.float32)
    if do_rotate:
        x = rotate(x, rotate_signs)
    B, H, N, d = x.shape
    nb = -(-N // block_rows)
    codes = np.empty(x.shape, np.uint8)
    desc = np.empty((B, H, nb), np.float32)
    for i in range(nb):
        blk = x[:, :, i * block_rows:(i + 1) * block_rows, :].astype(np.float64)
        ds = pow2_descale(np.abs(blk).max(axis=(2, 3)))
        desc[:, :, i] = ds
        y = np.clip(blk / ds.astype(np.float64)[:, :, None, None], -E4M3_MAX, E4M3_MAX)  # exact
        codes[:, :, i * block_rows:(i + 1) * block_rows, :] = e4m3_encode(y)
    return codes, desc


def dequantize_blocks(codes, desc, block_rows: int = 128) -> np.ndarray:
    """Inverse of quantize_blocks up to rounding: fp64 values code * descale."""
    vals = e4m3_decode(codes)
    N = vals.shape[2]
    scale = np.repeat(np.asarray(desc, np.float64), block_rows, axis=2)[:, :, :N]
    return vals * scale[..., None]
