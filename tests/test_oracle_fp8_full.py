"""Pins of the oracle's "fp8" precision: power-of-two V scales and E4M3
probabilities quantised before the row sum, each row with the same
power-of-two block scale rule as V.

The scale exponent is checked against a linear search; the V quantiser by
exact round trips of E4M3-representable blocks; the probability rounding by a
brute-force nearest-code search over the E4M3 value table (an independent
statement of round-to-nearest-even) with the row's scale exponent found by
linear search, inside a pure-Python attention loop, and by closed forms that
tell apart the plausible mistakes: no rounding, a scale that is not a power
of two (the exact row maximum as the reference), a scale one binade off, and
normalising by the unquantised sum.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.attention import attention_block, attention_block_fp8p
from oracle.fp8 import (E4M3_MAX, e4m3_decode, e4m3_encode, e4m3_round, pow2_scale_exponent,
                        quantize_blocks_pow2)
from oracle.geometry import Geometry, plan

# All finite non-negative E4M3 values with their codes (0x00..0x7e).
_CODES = np.arange(0, 0x7F, dtype=np.uint8)
_VALUES = e4m3_decode(_CODES)


def _nearest_code_value(x: float) -> float:
    """Brute force: the E4M3 value nearest to x >= 0; on a tie the even code."""
    best, best_d = None, None
    for c, val in zip(_CODES.tolist(), _VALUES.tolist()):
        d = abs(val - x)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = (c, val), d
    return best[1]


def _exponent_by_search(a: float) -> int:
    if a == 0:
        return 0
    for e in range(-200, 200):
        if a <= 448.0 * 2.0 ** e:
            return min(max(e, -126), 127)
    raise AssertionError


def test_pow2_exponent_boundaries_and_search():
    for k in range(-30, 30):
        edge = 448.0 * 2.0 ** k
        assert pow2_scale_exponent(edge) == k
        assert pow2_scale_exponent(np.nextafter(edge, np.inf)) == k + 1
        assert pow2_scale_exponent(np.nextafter(edge, 0)) == k
    rng = np.random.default_rng(3)
    xs = np.exp(rng.uniform(-60, 60, 2000))
    got = pow2_scale_exponent(xs)
    assert all(int(g) == _exponent_by_search(float(x)) for g, x in zip(got, xs))
    assert pow2_scale_exponent(0.0) == 0
    assert pow2_scale_exponent(1e-42) == -126      # clamped: sigma stays a normal float32
    assert pow2_scale_exponent(3.0e38) == 120


def test_quantize_pow2_round_trips_representable_blocks():
    g = Geometry(200, (5, 16, 24), True, 0.8, min_sparse_blocks=1)  # short head block
    p = plan(g)
    rng = np.random.default_rng(5)
    S, D = g.seq_len, 8
    codes = rng.integers(0, 0x7F, (1, 2, S, D)).astype(np.uint8)
    codes |= (rng.integers(0, 2, codes.shape) << 7).astype(np.uint8)    # random signs
    x = e4m3_decode(codes)
    ks = rng.integers(-20, 20, (2, p.n_blocks))
    for j, (r0, n) in enumerate(p.blocks):
        for h in range(2):
            x[0, h, r0, 0] = 320.0                                      # a value in (224, 448]
            x[0, h, r0:r0 + n] *= 2.0 ** ks[h, j]
    r0z, nz = p.blocks[3]
    x[0, 1, r0z:r0z + nz] = 0.0                                         # an all-zero block
    q8, sigma = quantize_blocks_pow2(x.astype(np.float32), p)
    for j, (r0, n) in enumerate(p.blocks):
        for h in range(2):
            if h == 1 and j == 3:
                assert sigma[0, h, j] == 1.0 and np.all(q8[0, h, r0:r0 + n] == 0)
                continue
            assert sigma[0, h, j] == 2.0 ** ks[h, j]
            deq = e4m3_decode(q8[0, h, r0:r0 + n]) * float(sigma[0, h, j])
            assert np.array_equal(deq, x[0, h, r0:r0 + n])


def test_quantize_pow2_error_and_range():
    g = Geometry(128, (9, 16, 32), True, 0.8)
    p = plan(g)
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((1, 2, g.seq_len, 16)) * 3).astype(np.float32)
    q8, sigma = quantize_blocks_pow2(x, p)
    for j, (r0, n) in enumerate(p.blocks):
        for h in range(2):
            sig = float(sigma[0, h, j])
            assert math.log2(sig) == int(math.log2(sig))                  # a power of two
            blk = x[0, h, r0:r0 + n].astype(np.float64)
            assert 224.0 < np.abs(blk).max() / sig <= 448.0                # before rounding
            top = np.abs(e4m3_decode(q8[0, h, r0:r0 + n])).max()
            assert 224.0 <= top <= 448.0
            err = np.abs(e4m3_decode(q8[0, h, r0:r0 + n]) * sig - blk)
            assert np.all(err <= np.maximum(np.abs(blk) * 2.0 ** -4, 2.0 ** -10 * sig))


def _fp8p_by_loops(q, k, v, scale):
    """Pure-Python statement of the reading, with brute-force rounding: the
    row's exponentials 2^t get the smallest power-of-two scale 2^e with
    max 2^t <= 448 * 2^e (found by search), then E4M3 codes."""
    out = []
    for qi in q:
        t = [scale / math.log(2.0) * sum(a * b for a, b in zip(qi, kc)) for kc in k]
        top = 2.0 ** max(t)
        e = next(e for e in range(-300, 300) if top <= 448.0 * 2.0 ** e)
        pq = [_nearest_code_value(2.0 ** (tc - e)) for tc in t]
        den = sum(pq)
        out.append([sum(pq[c] * v[c][d] for c in range(len(k))) / den for d in range(len(v[0]))])
    return np.array(out)


def test_fp8p_brute_force_small():
    rng = np.random.default_rng(7)
    for L in (1, 2, 5, 37):
        q = rng.standard_normal((3, 4)) * 2
        k = rng.standard_normal((L, 4)) * 2
        v = rng.standard_normal((L, 3))
        got = attention_block_fp8p(q, k, v, 0.5)
        ref = _fp8p_by_loops(q.tolist(), k.tolist(), v.tolist(), 0.5)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def _two_keys(t0, t1, v):
    """Attention of q = [1] over keys whose log2 logits are t0, t1 (scale = ln 2)."""
    return attention_block_fp8p(np.array([[1.0]]), np.array([[t0], [t1]]), v, math.log(2.0))[0]


def test_fp8p_closed_forms():
    v = np.array([[1.0, -2.0], [5.0, 7.0]])
    # Equal logits: every P is 256 (the scale 2^-8 puts 2^0 at 256 <= 448), the
    # output is the mean.
    np.testing.assert_allclose(
        attention_block_fp8p(np.zeros((1, 3)), np.ones((4, 3)), np.arange(8.0).reshape(4, 2), 1.0),
        [[3.0, 4.0]], atol=1e-15)
    # Integer logits: exact powers of two.
    np.testing.assert_allclose(_two_keys(3.0, 2.0, v), (v[0] + 0.5 * v[1]) / 1.5, atol=1e-15)
    # 256 * 0.95 = 243.2 rounds to 240 (step 16 in [128, 256)), and the row sum is
    # the sum of the rounded values: 256 and 240.
    np.testing.assert_allclose(_two_keys(0.0, math.log2(0.95), v),
                               (256 * v[0] + 240 * v[1]) / 496, atol=1e-15)
    # A power-of-two scale, the smallest that fits: max 2^2.3 <= 448 * 2^-6 (not
    # 2^-7), so P = (2^8.3, 2^6) = (315.2, 64) -> (320, 64). With the exact
    # maximum as the reference (a scale that is not a power of two) it would be
    # (2^8, 2^5.7) -> (256, 52).
    np.testing.assert_allclose(_two_keys(2.3, 0.0, v), (320 * v[0] + 64 * v[1]) / 384, atol=1e-15)
    # The scale exponent is the smallest that fits: 2^0.5 * 2^8 = 362 <= 448, so
    # e = -8 and a key 15.2 below gets 2^-6.7 = 0.0096, subnormal (below 2^-6),
    # rounded to 5 * 2^-9; a scale one binade lower (largest P in (112, 224])
    # would give 2^-7.7 -> 2 * 2^-9 instead. 2^8.5 = 362.04 rounds to 352 (step 32).
    np.testing.assert_allclose(_two_keys(0.5, -14.7, v),
                               (352 * v[0] + 5 * 2.0 ** -9 * v[1]) / (352 + 5 * 2.0 ** -9),
                               atol=1e-15)
    # A key 9.5 below the largest (P = 256) gets 2^-1.5 = 0.354, a normal value
    # that rounds to 11/32; with the largest P at 1 it would be subnormal and
    # round to 2^-9.
    np.testing.assert_allclose(_two_keys(0.0, -9.5, v),
                               (256 * v[0] + (11 / 32) * v[1]) / (256 + 11 / 32), atol=1e-15)
    # Subnormal P (below 2^-6): 2^-7 is exact, 2^-9.5 rounds to 2^-9, 2^-11 to 0.
    np.testing.assert_allclose(_two_keys(0.0, -15.0, v),
                               (256 * v[0] + 2.0 ** -7 * v[1]) / (256 + 2.0 ** -7), atol=1e-15)
    np.testing.assert_allclose(_two_keys(0.0, -17.5, v),
                               (256 * v[0] + 2.0 ** -9 * v[1]) / (256 + 2.0 ** -9), atol=1e-15)
    np.testing.assert_allclose(_two_keys(0.0, -19.0, v), v[0], atol=0)
    # Shifting every logit by an integer scales every P by the same power of two.
    for shift in (-40, 7, 300):
        np.testing.assert_allclose(_two_keys(2.3 + shift, shift, v), _two_keys(2.3, 0.0, v),
                                   atol=1e-15)
    # No keys: zeros.
    assert np.all(attention_block_fp8p(np.ones((2, 3)), np.zeros((0, 3)), np.zeros((0, 4)), 1.0) == 0)


def test_fp8p_scale_exponent_edges():
    """e = ceil(max t - log2 448): the largest exponential lands in (224, 448]."""
    from oracle.attention import fp8p_scale_exponent
    for k in range(-20, 20):
        # Just under 448 * 2^k fits that scale; just over it needs the next one.
        # (log2 448 is irrational: no float lands on the edge itself.)
        t = np.array([[math.log2(448.0) + k - 1e-9, -100.0]])
        assert fp8p_scale_exponent(t)[0, 0] == k
        t2 = np.array([[math.log2(448.0) + k + 1e-9, -100.0]])
        assert fp8p_scale_exponent(t2)[0, 0] == k + 1
    rng = np.random.default_rng(12)
    t = rng.uniform(-50, 50, (200, 7))
    e = fp8p_scale_exponent(t)
    top = np.exp2(t.max(axis=1, keepdims=True) - e)
    assert np.all((top > 224.0) & (top <= 448.0 * (1 + 1e-12)))


def test_fp8p_within_rounding_bound_of_exact_softmax():
    # |O_q - O| = |sum (P~ - P)(v - O)| / sum P~ <= max|v - O| * sum max(2^-4 P, 2^-10) / sum P~
    # with P = 2^(t - e), e = ceil(max t - log2 448), and half an E4M3 quantum per element.
    rng = np.random.default_rng(8)
    q = rng.standard_normal((16, 32))
    k = rng.standard_normal((300, 32))
    v = rng.standard_normal((300, 8))
    scale = 1 / math.sqrt(32)
    exact = attention_block(q, k, v, scale)
    quant = attention_block_fp8p(q, k, v, scale)
    t = scale / math.log(2.0) * (q @ k.T)
    pe = np.exp2(t - np.ceil(t.max(axis=1, keepdims=True) - math.log2(448.0)))
    pq = e4m3_round(pe)
    assert np.all(np.abs(pq - pe) <= np.maximum(pe * 2.0 ** -4, 2.0 ** -10))
    spread = np.abs(v[None, :, :] - exact[:, None, :]).max(axis=1)        # [16, 8]
    bound = spread * (np.maximum(pe * 2.0 ** -4, 2.0 ** -10).sum(axis=1) / pq.sum(axis=1))[:, None]
    assert np.all(np.abs(quant - exact) <= bound * (1 + 1e-12))
    assert np.abs(quant - exact).max() > 0                                # it does quantise


def test_fp8_pipeline_wiring():
    g = Geometry(128, (9, 16, 32), True, 0.8)
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((1, 2, g.seq_len, 16)).astype(np.float32) for _ in range(3))
    f = oracle.run(q, k, v, g, precision="fp8")
    m = oracle.run(q, k, v, g, precision="mix")
    # Q/K quantisation and selection as in mix.
    assert np.array_equal(f["q8"], m["q8"]) and np.array_equal(f["k_scale"], m["k_scale"])
    assert np.array_equal(f["select_idx"], m["select_idx"])
    p = f["plan"]
    deq = {}
    for name, codes, sig in (("q", f["q8"], f["q_scale"]), ("k", f["k8"], f["k_scale"]),
                             ("v", f["v8"], f["v_scale"])):
        d = np.empty(codes.shape)
        for j, (r0, n) in enumerate(p.blocks):
            d[:, :, r0:r0 + n] = e4m3_decode(codes[:, :, r0:r0 + n]) * sig[:, :, j, None, None]
        deq[name] = d
    ref = oracle.sparse_attention(deq["q"], deq["k"], deq["v"], p, f["select_idx"], f["select_num"],
                                  f["scale"], quantize_p=True)
    np.testing.assert_allclose(f["out_p"], ref, rtol=0, atol=1e-13)
    # All-fp8 stays close to the mix result.
    assert np.abs(f["out"] - m["out"]).max() < 6e-2
