"""Per-element bounds for the quantised precisions (fp8 and mxfp4), derived
from the code grids and each row's probability shares (test infrastructure;
numpy only).

fp8. ``kernel_bound`` bounds |GPU - oracle| where the oracle is the fp8
reading (``oracle.attention.attention_block_fp8p``) on the same E4M3 codes.
With ``x_c = 2^(t_c - e)`` the exact scaled exponentials and
``P_c = E4M3(x_c)``, a GPU probability can differ from ``P_c`` only in these
ways:

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
``|dO| <= sum_c |dP_c| |v_c - O| / (sum_c P_c - sum_c |dP_c|)``. The same
matrix product forms ``sum_c P_c v_c`` (and the row sum, as a product with an
all-ones operand) in steps of 64 keys of one block: 2^-10 of each step's
largest product, bounded per 32-key quarter of a block by the quarter's
largest P times its largest |v| (a step is two quarters). The GPU's fp32 sums
across steps add at most 1e-4 max|v| (a few hundred fp32 additions per row,
with a factor of three to spare), and rounding the output to bf16 at most half
an ulp, bounded here by 2^-8 |O|.

mxfp4. ``mx_kernel_bound`` bounds |GPU - attention_block_mxp| on the same
E2M1 codes and scales. The reading quantises ``x_c = 2^(t_c - ref)`` per MX
block of 32 keys (a quarter of a listed block) with the block's UOS scale 2^e
(the smallest e with max x <= 7.25 * 2^e) and E2M1 codes of x / 2^e. The
kernel's running integer reference and its per-lane scale shift x and 2^e by
the same power of two, so exact arithmetic gives the same codes; in the
GPU's fp32 a code differs only where:

* an element's x / 2^e lies within the relative error of an E2M1 midpoint;
* the block's largest x lies within that error of a scale boundary
  7.25 * 2^e or 7.25 * 2^(e - 1): the whole block may take the neighbouring
  scale.
For every element the bound takes the largest change over the candidate
scales and over both ends of x's error interval (the code is monotone in x),
and then the same output propagation and accumulation terms as fp8 (the
products are E2M1 times E2M1 with E8M0 scales, summed in the same 64-key
steps; the logit error model is the fp8 one).

``quant_bound`` bounds |reading - exact softmax attention| from the E4M3
rounding of P alone (the reading on dequantised Q/K/V against exact softmax on
the same operands): every P is within half a step of ``x_c``.
"""
from __future__ import annotations

import math

import numpy as np

from oracle.attention import fp8p_scale_exponent
from oracle.fp8 import e4m3_round
from oracle.mxfp4 import (MX_EXP_MIN, UOS_QMAX, e2m1_decode, e2m1_encode, mx_round_groups,
                          mx_scale_exponent)

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


def accumulation_error(P, v, groups):
    """Bound [M, D] on the matrix products' accumulation error in
    ``sum_c P_c v_c`` (numerator) and ``sum_c P_c`` (row sum), relative to the
    output: 2^-10 of each 64-key step's largest product, bounded per 32-key
    quarter (``groups``) by its largest P times its largest |v| per channel,
    and for the row sum by its largest P times |O|."""
    P = np.asarray(P, np.float64)
    av = np.abs(np.asarray(v, np.float64))
    pmax = np.stack([P[:, a:b].max(axis=1) for a, b in groups], axis=1)
    vmax = np.stack([av[a:b].max(axis=0) for a, b in groups], axis=0)
    den = P.sum(axis=1, keepdims=True)
    O = np.abs((P @ np.asarray(v, np.float64)) / den)
    return MATRIX_STEP_ERROR * ((pmax @ vmax) + pmax.sum(axis=1, keepdims=True) * O) / den


def _propagate(P, dP, v, groups):
    """Output bound [M, D] from probability changes ``dP`` (per key) and the
    products' accumulation and rounding (see the module docstring)."""
    den = P.sum(axis=1, keepdims=True)
    O = (P @ v) / den
    spread = np.empty_like(O)
    for r in range(P.shape[0]):
        nz = dP[r] > 0
        spread[r] = (dP[r, nz, None] * np.abs(v[nz] - O[r])).sum(axis=0) if nz.any() else 0.0
    shift = spread / np.maximum(den - dP.sum(axis=1, keepdims=True), 1e-300)
    return (shift + accumulation_error(P, v, groups) + 2.0 ** -8 * np.abs(O)
            + 1e-4 * np.abs(v).max() + 1e-7)


def kernel_bound(q, k, v, scale, groups):
    """Per-element bound [M, D] of |GPU - attention_block_fp8p(q, k, v, scale)|
    for query rows ``q [M, D]`` over keys ``k, v [L, D]`` (dequantised);
    ``groups``: the 32-key quarters of the listed blocks
    (``oracle.attention.listed_groups``)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    if k.shape[0] == 0:
        return np.full((q.shape[0], v.shape[1]), 1e-7)
    t, e, x = _scaled_exponentials(q, k, scale)
    P = e4m3_round(x)
    dP = np.where(flip_candidates(q, k, scale), _step(x), 0.0)
    dP = np.where(x < SUBNORMAL_MIN_NORMAL, SUBNORMAL_STEP, dP)
    return _propagate(P, dP, v, groups)


def _mx_value(x, e):
    """The MXFP4 value of x >= 0 at scale exponent e (per row, broadcast)."""
    s = np.exp2(np.asarray(e, np.float64))
    return e2m1_decode(e2m1_encode(x / s)) * s


def mx_relative_error(q, k, scale):
    """Bound [M, L] on the relative error of the GPU's scaled exponentials in
    mxfp4: the logit error (as fp8) plus fp32 rounding of the scale product
    and of the fused add of the integer exponents (the running reference and
    the block scale, which can sit up to twice the row's largest |t| away),
    and exp2's."""
    t = (scale / math.log(2.0)) * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    ref = np.ceil(t.max(axis=1, keepdims=True))
    big = np.abs(t).max(axis=1, keepdims=True)
    dt = logit_error(q, k, scale) + 2.0 ** -21 * (np.abs(t) + np.abs(t - ref) + 2 * big + 16)
    return t, ref, math.log(2.0) * dt + 2.0 ** -20


def mx_kernel_bound(q, k, v, scale, groups):
    """Per-element bound [M, D] of |GPU - attention_block_mxp(q, k, v, scale,
    groups)| for query rows ``q [M, D]`` over keys ``k, v [L, D]``
    (dequantised), ``groups`` the MX blocks of P (32-key quarters)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    if k.shape[0] == 0:
        return np.full((q.shape[0], v.shape[1]), 1e-7)
    t, ref, rel = mx_relative_error(q, k, scale)
    x = np.exp2(t - ref)
    P = mx_round_groups(x, groups)
    dP = np.zeros_like(P)
    for a, b in groups:
        xg, rg, pg = x[:, a:b], rel[:, a:b], P[:, a:b]
        amax = xg.max(axis=1)
        rmax = rg.max(axis=1)
        e = mx_scale_exponent(amax).astype(np.float64)
        lo_x, hi_x = xg * (1.0 - rg), xg * (1.0 + rg)
        worst = np.zeros_like(pg)
        for de, can in ((0, np.ones_like(amax, dtype=bool)),
                        (-1, amax * (1.0 - rmax) <= UOS_QMAX * np.exp2(e - 1)),
                        (1, amax * (1.0 + rmax) > UOS_QMAX * np.exp2(e))):
            if not can.any():
                continue
            ee = (e + de)[:, None]
            d = np.maximum(np.abs(_mx_value(lo_x, ee) - pg), np.abs(_mx_value(hi_x, ee) - pg))
            worst = np.where(can[:, None], np.maximum(worst, d), worst)
        # A block at the smallest E8M0 scale (values below 2^-124): any code.
        tiny = e <= MX_EXP_MIN + 1
        worst = np.where(tiny[:, None], np.maximum(worst, pg + hi_x), worst)
        dP[:, a:b] = worst
    return _propagate(P, dP, v, groups)


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
