"""OCP FP8 E4M3 codec and the per-block quantisation of the "mix" and "fp8" precisions.

TEST INFRASTRUCTURE (see the package docstring).

The pages name a kernel precision "mix" ("RainFusion Attention",
Configuration: ``precision`` is ``"bf16"``, ``"fp8"`` or ``"mix"``) but do
not define it. Reading: Q and K are stored as fp8 E4M3 with one float32 scale
per 128-row block of the permuted sequence (short blocks included) and per
head; V, the probabilities and the output stay bf16; softmax is float32.

E4M3 (OCP 8-bit floating point specification): 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits; exponent field 0 holds subnormals
``m * 2**-9``; the largest finite magnitude is 448 (exponent field 15,
mantissa 6); exponent field 15 with mantissa 7 is NaN; there are no
infinities. Encoding rounds to nearest with ties to even and saturates
finite values beyond 448 to +-448.

Per-block scale (the float32 steps decide the integer codes, so they are
fixed here and the GPU path does the same float32 operations):

* ``amax`` = largest |x| over the block's rows and channels (exact);
* ``r = float32(448) / amax`` (one correctly-rounded float32 division);
* ``code = e4m3(float32(x * r))`` (one correctly-rounded float32 multiply);
* stored scale ``sigma = amax / float32(448)`` (float32 division);
* an all-zero block uses ``r = sigma = 1``.

The dequantised value is ``decode(code) * sigma``.

The "fp8" precision (same Configuration row, equally undefined there) is read
as every attention operand in E4M3: Q and K exactly as in "mix"; V per
(batch, kv head, 128-row block) with a power-of-two scale (below); and the
probabilities P as E4M3 codes of the unnormalised exponentials, each row
quantised with the same power-of-two block scale rule as V (``attention.py``).

Power-of-two block scale (V in "fp8"): ``sigma = 2**e`` with ``e`` the
smallest integer such that ``amax <= 448 * 2**e``, clamped to [-126, 127]
(so sigma is a normal float32); an all-zero block uses ``e = 0``. Then
``code = e4m3(x / sigma)``: dividing by a power of two is exact, so the codes
depend on the values alone, and the block's largest magnitude lands in
(224, 448]. A power-of-two scale is what the gfx950 scaled fp8 products take
as a per-operand block exponent (E8M0), so the kernel applies it exactly.
"""
from __future__ import annotations

import numpy as np

from .geometry import Plan

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Finite float values -> uint8 E4M3 codes (round to nearest even, saturating)."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode takes finite values only")
    sign = np.signbit(x)
    a = np.abs(x)
    # Exponent of the binade holding a, clamped to the normal minimum 2**-6 so the
    # subnormal range keeps the fixed quantum 2**-9.
    _, ex = np.frexp(np.where(a > 0, a, 1.0))      # a = f * 2**ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)
    quantum = np.exp2(e - 3.0)                      # 3 mantissa bits
    steps = a / quantum                             # exact (power-of-two scaling)
    rounded = np.round(steps)                       # numpy rounds halves to even
    val = np.minimum(rounded * quantum, E4M3_MAX)   # saturate
    # Encode the (exactly representable) value.
    _, vex = np.frexp(np.where(val > 0, val, 1.0))
    ve = vex - 1
    normal = val >= 2.0 ** -6
    efield = np.where(normal, ve + 7, 0)
    mfield = np.where(normal, val / np.exp2(ve.astype(np.float64)) * 8 - 8, val / 2.0 ** -9)
    code = (efield.astype(np.int64) << 3) | np.rint(mfield).astype(np.int64)
    code = np.where(val == 0, 0, code)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def quantize_blocks(xp_f32: np.ndarray, p: Plan):
    """Quantise permuted ``[B, N, S, D]`` float32 values per (batch, head, block).

    Returns ``(codes uint8 [B, N, S, D], sigma float32 [B, N, n_blocks])``.
    """
    x = np.asarray(xp_f32, dtype=np.float32)
    B, N, S, D = x.shape
    codes = np.zeros((B, N, S, D), dtype=np.uint8)
    sigma = np.ones((B, N, p.n_blocks), dtype=np.float32)
    for j, (r0, n) in enumerate(p.blocks):
        blk = x[:, :, r0:r0 + n, :]
        amax = np.abs(blk).max(axis=(2, 3)).astype(np.float32)          # [B, N]
        zero = amax == 0
        safe = np.where(zero, np.float32(1), amax)
        r = np.where(zero, np.float32(1), np.float32(E4M3_MAX) / safe).astype(np.float32)
        sig = np.where(zero, np.float32(1), safe / np.float32(E4M3_MAX)).astype(np.float32)
        y = (blk * r[:, :, None, None]).astype(np.float32)
        codes[:, :, r0:r0 + n, :] = e4m3_encode(y)
        sigma[:, :, j] = sig
    return codes, sigma


POW2_EXP_MIN, POW2_EXP_MAX = -126, 127


def pow2_scale_exponent(amax) -> np.ndarray:
    """Smallest integer ``e`` with ``amax <= 448 * 2**e`` (clamped to [-126, 127]);
    0 where ``amax == 0``. The estimate from log2 is corrected by exact float64
    comparisons (``448 * 2**e`` is exact), so the result is exact."""
    a = np.asarray(amax, dtype=np.float64)
    pos = a > 0
    e = np.ceil(np.log2(np.where(pos, a, E4M3_MAX) / E4M3_MAX))
    e = np.where(E4M3_MAX * np.exp2(e) < a, e + 1, e)           # too small: step up
    e = np.where(E4M3_MAX * np.exp2(e - 1) >= a, e - 1, e)      # not the smallest: step down
    e = np.where(pos, e, 0)
    return np.clip(e, POW2_EXP_MIN, POW2_EXP_MAX).astype(np.int64)


def quantize_blocks_pow2(xp_f32: np.ndarray, p: Plan):
    """Quantise permuted ``[B, N, S, D]`` values per (batch, head, block) with a
    power-of-two scale. Returns ``(codes uint8 [B, N, S, D], sigma float32 [B, N, n_blocks])``."""
    x = np.asarray(xp_f32, dtype=np.float64)
    B, N, S, D = x.shape
    codes = np.zeros((B, N, S, D), dtype=np.uint8)
    sigma = np.ones((B, N, p.n_blocks), dtype=np.float32)
    for j, (r0, n) in enumerate(p.blocks):
        blk = x[:, :, r0:r0 + n, :]
        amax = np.abs(blk).max(axis=(2, 3))                              # [B, N]
        sig = np.exp2(pow2_scale_exponent(amax).astype(np.float64))     # [B, N]
        codes[:, :, r0:r0 + n, :] = e4m3_encode(blk / sig[:, :, None, None])
        sigma[:, :, j] = sig.astype(np.float32)
    return codes, sigma


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Values rounded to E4M3 (nearest, ties to even, saturating): decode(encode(x))."""
    return e4m3_decode(e4m3_encode(x))
