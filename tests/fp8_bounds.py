"""Per-element bounds for the fp8 precision, derived from the E4M3 quantum and
each row's probability shares (test infrastructure; numpy only).

``kernel_bound`` bounds |GPU - oracle| where the oracle is the fp8 reading
(``oracle.attention.attention_block_fp8p``) on the same E4M3 codes. With
``x_c = 2^(t_c - e)`` the exact scaled exponentials and ``P_c = E4M3(x_c)``,
a GPU probability can differ from ``P_c`` only in these ways:

* ``x_c`` lies within the relative error of the GPU's logits and
  exponentials of an E4M3 rounding midpoint: the code may be the neighbour,
  one E4M3 step of ``x_c``'s binade. The logits come from gfx950's scaled
  fp8 matrix product, which sums each 64-channel step's products with an
  error of up to 2^-11.4 of the step's largest product (measured on MI355X:
  exact when the products share a narrow exponent range; 2^-11.4 at most over
  13,000 wide-range trials); the bound takes 2^-10 of the largest product per
  step, plus fp32 rounding of the scale, the exponent and exp2;
* ``x_c`` is subnormal (below 2^-6): a one-pass kernel rounds earlier blocks
  at a smaller scale exponent, on a finer grid, and the two results differ by
  at most one subnormal step, 2^-9;
* every other code is the same.
With ``O`` the reading's output, changing P by ``dP`` moves the output by
``sum_c dP_c (v_c - O) / sum_c (P_c + dP_c)``, so per channel
``|dO| <= sum_c |dP_c| |v_c - O| / (sum_c P_c - sum_c |dP_c|)``. The GPU's
fp32 sums add at most 1e-4 max|v| (a few hundred fp32 additions per row, with
a factor of three to spare), and rounding the output to bf16 at most half an
ulp, bounded here by 2^-8 |O|.

``quant_bound`` bounds |reading - exact softmax attention| from the E4M3
rounding of P alone (the reading on dequantised Q/K/V against exact softmax on
the same operands): every P is within half a step of ``x_c``.
"""
from __future__ import annotations

import math

import numpy as np

from oracle.attention import fp8p_scale_exponent
from oracle.fp8 import e4m3_round

SUBNORMAL_MIN_NORMAL = 2.0 ** -6
SUBNORMAL_STEP = 2.0 ** -9


def _scaled_exponentials(q, k, scale):
    t = (scale / math.log(2.0)) * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    e = fp8p_scale_exponent(t)
    return t, e, np.exp2(t - e)


def _step(x):
    """E4M3 step (distance between neighbouring codes) at each value x >= 0."""
    xs = np.where(x > 0, x, 1.0)
    return np.where(x < SUBNORMAL_MIN_NORMAL, SUBNORMAL_STEP,
                    np.exp2(np.floor(np.log2(xs)) - 3.0))


MATRIX_STEP = 64                 # channels per fp8 matrix-product step
MATRIX_STEP_ERROR = 2.0 ** -10   # of the step's largest |q_i k_i| (measured max 2^-11.4)


def logit_error(q, k, scale):
    """Bound [M, L] on the GPU's logit error in log2 units: per 64-channel
    step of the fp8 product, MATRIX_STEP_ERROR times the step's largest
    |q_i k_i|, itself bounded by max_i |q_i| * max_i |k_i| over the step,
    after the scale."""
    q = np.abs(np.asarray(q, np.float64))
    k = np.abs(np.asarray(k, np.float64))
    D = q.shape[1]
    err = np.zeros((q.shape[0], k.shape[0]))
    for s0 in range(0, D, MATRIX_STEP):
        err += np.outer(q[:, s0:s0 + MATRIX_STEP].max(axis=1), k[:, s0:s0 + MATRIX_STEP].max(axis=1))
    return (scale / math.log(2.0)) * MATRIX_STEP_ERROR * err


def flip_candidates(q, k, scale):
    """Boolean [M, L]: keys whose scaled exponential lies within the GPU's
    relative error of an E4M3 rounding midpoint (normal range only).

    The relative error of the GPU's exponential: ln 2 times the logit error
    (``logit_error``, plus fp32 rounding of the scale product and the fused
    add of the exponent, 2^-22 |t| each, taken twice over) plus exp2's (2^-21)."""
    t, e, x = _scaled_exponentials(q, k, scale)
    dt = logit_error(q, k, scale) + 2.0 ** -21 * (np.abs(t) + np.abs(t - e))
    rel = math.log(2.0) * dt + 2.0 ** -20
    step = _step(x)
    lo = np.floor(x / step) * step
    mid = lo + 0.5 * step
    return (x >= SUBNORMAL_MIN_NORMAL) & (np.abs(x - mid) <= rel * x)


def kernel_bound(q, k, v, scale):
    """Per-element bound [M, D] of |GPU - attention_block_fp8p(q, k, v, scale)|
    for query rows ``q [M, D]`` over keys ``k, v [L, D]`` (dequantised)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    if k.shape[0] == 0:
        return np.full((q.shape[0], v.shape[1]), 1e-7)
    t, e, x = _scaled_exponentials(q, k, scale)
    P = e4m3_round(x)
    den = P.sum(axis=1, keepdims=True)
    O = (P @ v) / den
    dP = np.where(flip_candidates(q, k, scale), _step(x), 0.0)
    dP = np.where(x < SUBNORMAL_MIN_NORMAL, SUBNORMAL_STEP, dP)
    # sum_c dP_c |v_c - O| per row and channel, without forming [M, L, D].
    spread = np.empty_like(O)
    for r in range(q.shape[0]):
        nz = dP[r] > 0
        spread[r] = (dP[r, nz, None] * np.abs(v[nz] - O[r])).sum(axis=0) if nz.any() else 0.0
    shift = spread / np.maximum(den - dP.sum(axis=1, keepdims=True), 1e-300)
    return shift + 2.0 ** -8 * np.abs(O) + 1e-4 * np.abs(v).max() + 1e-7


def quant_bound(q, k, v, scale):
    """Per-element bound [M, D] of |attention_block_fp8p - exact softmax
    attention| on the same (dequantised) operands: half an E4M3 step per P."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    t, e, x = _scaled_exponentials(q, k, scale)
    P = e4m3_round(x)
    O = (x @ v) / x.sum(axis=1, keepdims=True)
    half = 0.5 * _step(x)
    spread = np.empty_like(O)
    for r in range(q.shape[0]):
        spread[r] = half[r] @ np.abs(v - O[r])
    return spread / P.sum(axis=1, keepdims=True) + 1e-12
