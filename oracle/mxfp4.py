"""OCP MXFP4 codec, the "mxfp4" precision's quantisers, and its scale rule.

TEST INFRASTRUCTURE (see the package docstring).

"RainFusion Attention" (Wan2.2 T2V quantization) lets the block-sparse path
run in ``mxfp4`` as well as ``fp8`` and passes the precision straight to the
native operator; it says the quantised paths keep the library's "default
rotation policy" and defines neither. "MXAttention: Data-Free Optimal Scaling
and Pre-Normalization Quantization for MXFP4 Attention" (abstract) gives the
two parts that are defined: a power-of-two scaling boundary Qmax = 7.25
(Universal Optimal Scaling) and quantising the unnormalised softmax
exponentials before the row sum (Pre-Normalization Quantization).

Readings (the plainest that the rest supports):

* MXFP4 is the OCP microscaling format: blocks of 32 consecutive elements along
  the dimension a product contracts, each element E2M1, one shared power-of-two
  scale per block (an E8M0 exponent, 2**-127 .. 2**127).
* Scale (UOS): ``2**e`` with ``e`` the smallest integer such that
  ``amax <= 7.25 * 2**e`` (clamped to [-127, 127]; an all-zero block gets
  -127, the clamp of -inf). The block's largest magnitude then lies in
  (3.625, 7.25] before rounding; values above 6 saturate to 6.
* Elements: ``code = E2M1(x / 2**e)``, nearest with ties to the even code,
  saturating at +-6. Dividing by a power of two is exact, so the codes depend
  on the values alone.
* Q and K: blocks of 32 channels of each row. V: blocks of 32 consecutive keys
  of one channel, the four quarters of each 128-row block of the arranged
  sequence (a short block's quarters hold its real rows only). P: the same key
  quarters, per query row (``attention.py``).
* Rotation: none (the "default rotation policy" is not defined on the pages).

E2M1 (OCP MX specification): 1 sign bit, 2 exponent bits with bias 1, 1
mantissa bit; exponent field 0 is subnormal (``m * 0.5``); magnitudes
0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN.
"""
from __future__ import annotations

import numpy as np

from .geometry import Plan

E2M1_MAX = 6.0
UOS_QMAX = 7.25
MX_BLOCK = 32
MX_EXP_MIN, MX_EXP_MAX = -127, 127


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit codes (0..15, sign in bit 3) -> float64 values."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return sign * mag


def e2m1_encode(x: np.ndarray) -> np.ndarray:
    """Finite values -> uint8 E2M1 codes: nearest, ties to even, saturating at +-6.

    The spacing of the values is 0.5 below 2 (the subnormals 0, 0.5 and the
    binade [1, 2)), 1 in [2, 4) and 2 from 4 on; the magnitude is rounded to a
    whole number of that quantum (halves to even, which is the even code),
    then capped at 6."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e2m1_encode takes finite values only")
    a = np.abs(x)
    quantum = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    val = np.minimum(np.round(a / quantum) * quantum, E2M1_MAX)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    code = np.searchsorted(mags, val)                  # val is exactly one of mags
    # The sign survives rounding, also to zero (-0.25 -> -0, code 8).
    return (code | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def e2m1_round(x: np.ndarray) -> np.ndarray:
    """Values rounded to E2M1: decode(encode(x))."""
    return e2m1_decode(e2m1_encode(x))


def mx_scale_exponent(amax) -> np.ndarray:
    """UOS: smallest integer ``e`` with ``amax <= 7.25 * 2**e``, clamped to
    [-127, 127] (-127 for ``amax == 0``). The log2 estimate is corrected by
    exact float64 comparisons (``7.25 * 2**e`` is exact)."""
    a = np.asarray(amax, dtype=np.float64)
    pos = a > 0
    e = np.ceil(np.log2(np.where(pos, a, UOS_QMAX) / UOS_QMAX))
    e = np.where(UOS_QMAX * np.exp2(e) < a, e + 1, e)
    e = np.where(UOS_QMAX * np.exp2(e - 1) >= a, e - 1, e)
    e = np.where(pos, e, MX_EXP_MIN)
    return np.clip(e, MX_EXP_MIN, MX_EXP_MAX).astype(np.int64)


def mx_quantize_group(x: np.ndarray):
    """One MX block (any length <= 32, along the last axis of ``x``).

    Returns ``(codes uint8, e int)`` with ``e`` over the leading axes."""
    x = np.asarray(x, dtype=np.float64)
    e = mx_scale_exponent(np.abs(x).max(axis=-1)) if x.shape[-1] else np.full(x.shape[:-1], MX_EXP_MIN)
    return e2m1_encode(x / np.exp2(e.astype(np.float64))[..., None]), e


def quantize_rows_mx(xp: np.ndarray):
    """Q or K: ``[B, N, S, D]`` -> codes ``[B, N, S, D]``, exponents ``[B, N, S, D/32]``
    (block c covers channels [32 c, 32 c + 32))."""
    x = np.asarray(xp, dtype=np.float64)
    B, N, S, D = x.shape
    if D % MX_BLOCK:
        raise ValueError("head_dim must be a multiple of 32")
    g = x.reshape(B, N, S, D // MX_BLOCK, MX_BLOCK)
    codes, e = mx_quantize_group(g)
    return codes.reshape(B, N, S, D), e


def dequantize_rows_mx(codes: np.ndarray, e: np.ndarray) -> np.ndarray:
    B, N, S, D = codes.shape
    v = e2m1_decode(codes).reshape(B, N, S, D // MX_BLOCK, MX_BLOCK)
    return (v * np.exp2(e.astype(np.float64))[..., None]).reshape(B, N, S, D)


def quantize_v_mx(vp: np.ndarray, p: Plan):
    """V: ``[B, N, S, D]`` (arranged rows) -> codes ``[B, N, S, D]`` and exponents
    ``[B, N, n_blocks, 4, D]``: quarter g of block j covers its real rows
    [32 g, 32 g + 32); a quarter past the block's end has no rows (-127)."""
    x = np.asarray(vp, dtype=np.float64)
    B, N, S, D = x.shape
    codes = np.zeros((B, N, S, D), dtype=np.uint8)
    e = np.full((B, N, p.n_blocks, 4, D), MX_EXP_MIN, dtype=np.int64)
    for j, (r0, n) in enumerate(p.blocks):
        for g in range(4):
            a, b = r0 + MX_BLOCK * g, r0 + min(MX_BLOCK * (g + 1), n)
            if a >= b:
                continue
            blk = np.swapaxes(x[:, :, a:b, :], 2, 3)                     # [B, N, D, rows]
            c, eg = mx_quantize_group(blk)
            codes[:, :, a:b, :] = np.swapaxes(c, 2, 3)
            e[:, :, j, g, :] = eg
    return codes, e


def dequantize_v_mx(codes: np.ndarray, e: np.ndarray, p: Plan) -> np.ndarray:
    out = e2m1_decode(codes)
    for j, (r0, n) in enumerate(p.blocks):
        for g in range(4):
            a, b = r0 + MX_BLOCK * g, r0 + min(MX_BLOCK * (g + 1), n)
            if a < b:
                out[:, :, a:b, :] *= np.exp2(e[:, :, j, g, :].astype(np.float64))[:, :, None, :]
    return out


def mx_round_groups(x: np.ndarray, groups) -> np.ndarray:
    """Rows ``x [M, L]`` quantised to MXFP4 and dequantised, one MX block per
    ``(start, stop)`` column range in ``groups`` (ranges of at most 32)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    for a, b in groups:
        if not 0 < b - a <= MX_BLOCK:
            raise ValueError("an MX group holds 1 to 32 elements")
        c, e = mx_quantize_group(x[:, a:b])
        out[:, a:b] = e2m1_decode(c) * np.exp2(e.astype(np.float64))[:, None]
    return out
