"""Pins of the oracle's "mxfp4" precision (MXFP4 with UOS scales; P quantised
before the row sum).

The E2M1 codec is checked against the format's value table and a brute-force
nearest-value search; the UOS exponent against a linear search and the cases
that tell 7.25 apart from the neighbouring boundaries (6, as a no-clipping
rule would use, and 8, the OCP floor rule); the quantisers by exact round
trips and the per-element error bound; the probability step by a pure-Python
loop with brute-force rounding and by closed forms that tell apart the
plausible mistakes: no rounding, one MX block across a group boundary, the
exact maximum instead of its integer ceiling as the reference, and
normalising by the unquantised sum.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.attention import attention_block, attention_block_mxp, listed_groups
from oracle.geometry import Geometry, plan
from oracle.mxfp4 import (dequantize_rows_mx, dequantize_v_mx, e2m1_decode, e2m1_encode,
                          e2m1_round, mx_round_groups, mx_scale_exponent, quantize_rows_mx,
                          quantize_v_mx)

# The E2M1 value table of the OCP MX specification, codes 0..15.
TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_decode_is_the_table():
    got = e2m1_decode(np.arange(16))
    assert got.tolist() == TABLE
    assert np.signbit(got[8])


def _nearest_code(x: float) -> int:
    """Brute force: the code whose value is nearest to x; ties to the even code;
    the sign of x kept (also for a zero result)."""
    best, best_d = None, None
    for c in range(8):
        d = abs(Fraction(TABLE[c]) - Fraction(abs(x)))            # exact distance
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best | (8 if math.copysign(1.0, x) < 0 else 0)


def test_encode_brute_force_grid():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0]
    xs = [0.0, -0.0, 1e-30, 6.0, 6.5, 7.25, 8.0, 100.0, 1e30]
    for m in mids:
        xs += [m, np.nextafter(m, 0), np.nextafter(m, np.inf)]
    xs += list(np.linspace(0, 9, 721))
    xs = np.array(xs + [-x for x in xs])
    got = e2m1_encode(xs)
    assert [int(c) for c in got] == [_nearest_code(float(x)) for x in xs]
    # Ties go to the even code: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2,
    # 3.5 -> 4, 5 -> 4; 7 lies between 6 and (unrepresentable) 8 and saturates to 6.
    np.testing.assert_array_equal(e2m1_round(np.array(mids)), [0, 1, 1, 2, 2, 4, 4, 6])


def _exp_by_search(a: float) -> int:
    if a == 0:
        return -127
    for e in range(-400, 400):
        if a <= 7.25 * 2.0 ** e:
            return min(max(e, -127), 127)
    raise AssertionError


def test_uos_exponent_boundaries_and_search():
    for k in range(-40, 40):
        edge = 7.25 * 2.0 ** k
        assert mx_scale_exponent(edge) == k
        assert mx_scale_exponent(np.nextafter(edge, np.inf)) == k + 1
        assert mx_scale_exponent(np.nextafter(edge, 0)) == k
    rng = np.random.default_rng(11)
    xs = np.exp(rng.uniform(-80, 80, 3000))
    assert all(int(g) == _exp_by_search(float(x)) for g, x in zip(mx_scale_exponent(xs), xs))
    assert mx_scale_exponent(0.0) == -127
    assert mx_scale_exponent(2.0 ** -140) == -127            # clamped to the E8M0 minimum
    assert mx_scale_exponent(3.0e38) == 125                   # 3e38 <= 7.25 * 2^125 = 3.08e38
    assert mx_scale_exponent(3.3e38) == 126


def test_uos_boundary_is_7_25():
    # [7.1, 0.6]: 7.1 <= 7.25, so e = 0: 7.1 -> 6, 0.6 -> 0.5. A boundary of 6
    # (no clipping) would take e = 1 and give 8 and 1.0.
    np.testing.assert_array_equal(mx_round_groups(np.array([[7.1, 0.6]]), [(0, 2)]), [[6.0, 0.5]])
    # [7.3, 0.6]: 7.3 > 7.25, so e = 1: 3.65 -> 4 -> 8, 0.3 -> 0.5 -> 1.0. The OCP
    # floor rule (largest element in [4, 8)) would keep e = 0 and give 6 and 0.5.
    np.testing.assert_array_equal(mx_round_groups(np.array([[7.3, 0.6]]), [(0, 2)]), [[8.0, 1.0]])
    # The scaled block maximum lies in (3.625, 7.25] before rounding.
    rng = np.random.default_rng(12)
    x = rng.standard_normal((500, 32)) * np.exp(rng.uniform(-20, 20, (500, 1)))
    e = mx_scale_exponent(np.abs(x).max(axis=1))
    top = np.abs(x).max(axis=1) / np.exp2(e.astype(float))
    assert np.all(top > 3.625) and np.all(top <= 7.25)


def _err_bound(x, e):
    """Half a quantum at |x| / 2**e (0.25 below 2, 0.5 below 4, 1 up to 6), or the
    clipping error above 6 (at most 1.25), times 2**e."""
    y = np.abs(x) / np.exp2(e)
    h = np.where(y < 2, 0.25, np.where(y < 4, 0.5, np.where(y <= 6, 1.0, y - 6)))
    return h * np.exp2(e)


def test_quantize_rows_round_trip_and_error():
    rng = np.random.default_rng(13)
    B, N, S, D = 1, 2, 50, 128
    codes = rng.integers(0, 16, (B, N, S, D)).astype(np.uint8)
    x = e2m1_decode(codes)
    ks = rng.integers(-30, 30, (B, N, S, D // 32))
    for c in range(D // 32):
        x[..., 32 * c] = 6.0 * np.where(rng.integers(0, 2, (B, N, S)) > 0, 1.0, -1.0)
        x[..., 32 * c:32 * c + 32] *= np.exp2(ks[..., c:c + 1].astype(float))
    c4, e4 = quantize_rows_mx(x)
    np.testing.assert_array_equal(e4, ks)
    np.testing.assert_array_equal(dequantize_rows_mx(c4, e4), x)
    # Random data: every element within its bound, the block scale from the block alone.
    y = rng.standard_normal((B, N, S, D)) * 3
    c4, e4 = quantize_rows_mx(y)
    err = np.abs(dequantize_rows_mx(c4, e4) - y)
    np.testing.assert_array_less(err, _err_bound(y, np.repeat(e4, 32, axis=-1)) * (1 + 1e-12) + 1e-300)
    y2 = y.copy()
    y2[..., 32:64] *= 1000.0                                  # another block: no effect here
    np.testing.assert_array_equal(quantize_rows_mx(y2)[0][..., :32], c4[..., :32])


def test_quantize_v_quarters_short_block():
    g = Geometry(200, (5, 16, 24), True, 0.8, min_sparse_blocks=1)   # head blocks 128 + 72 + ...
    p = plan(g)
    j_short = next(j for j, (r0, n) in enumerate(p.blocks) if n % 32 and n < 128)
    r0, n = p.blocks[j_short]
    rng = np.random.default_rng(14)
    S, D = g.seq_len, 64
    codes = rng.integers(0, 16, (1, 1, S, D)).astype(np.uint8)
    x = e2m1_decode(codes)
    kq = rng.integers(-10, 10, (p.n_blocks, 4, D))
    for j, (a0, m) in enumerate(p.blocks):
        for q in range(4):
            a, b = a0 + 32 * q, a0 + min(32 * q + 32, m)
            if a < b:
                x[0, 0, a, :] = 4.0                          # each quarter's maximum
                x[0, 0, a:b, :] *= np.exp2(kq[j, q].astype(float))
    c, e = quantize_v_mx(x, p)
    for j, (a0, m) in enumerate(p.blocks):
        for q in range(4):
            if 32 * q < m:
                np.testing.assert_array_equal(e[0, 0, j, q], kq[j, q])
            else:
                assert np.all(e[0, 0, j, q] == -127)        # no rows: the clamp of -inf
    np.testing.assert_array_equal(dequantize_v_mx(c, e, p), x)
    assert n % 32 != 0                                       # the partial quarter was covered


def _mx_by_loops(q, k, v, scale, groups):
    """Pure-Python statement of the reading with brute-force rounding."""
    out = []
    for qi in q:
        t = [scale / math.log(2.0) * sum(a * b for a, b in zip(qi, kc)) for kc in k]
        ref = math.ceil(max(t))
        x = [2.0 ** (tc - ref) for tc in t]
        pq = [0.0] * len(x)
        for a, b in groups:
            e = _exp_by_search(max(abs(y) for y in x[a:b]))
            for c in range(a, b):
                pq[c] = abs(TABLE[_nearest_code(x[c] / 2.0 ** e)]) * 2.0 ** e
        den = sum(pq)
        out.append([sum(pq[c] * v[c][d] for c in range(len(k))) / den for d in range(len(v[0]))])
    return np.array(out)


def test_mxp_brute_force_small():
    rng = np.random.default_rng(15)
    for L, groups in ((1, [(0, 1)]), (5, [(0, 5)]), (37, [(0, 32), (32, 37)]),
                      (70, [(0, 32), (32, 64), (64, 70)]), (40, [(0, 8), (8, 40)])):
        q = rng.standard_normal((3, 4)) * 2
        k = rng.standard_normal((L, 4)) * 2
        v = rng.standard_normal((L, 3))
        got = attention_block_mxp(q, k, v, 0.5, groups)
        ref = _mx_by_loops(q.tolist(), k.tolist(), v.tolist(), 0.5, groups)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def _keys(ts, v, groups):
    """Attention of q = [1] over keys whose log2 logits are ts (scale = ln 2)."""
    k = np.array(ts, dtype=float)[:, None]
    return attention_block_mxp(np.array([[1.0]]), k, v, math.log(2.0), groups)[0]


def test_mxp_closed_forms():
    v = np.array([[1.0, -2.0], [5.0, 7.0]])
    # Equal logits: equal P, the output is the mean.
    np.testing.assert_allclose(_keys([0.4] * 4, np.arange(8.0).reshape(4, 2), [(0, 4)]),
                               [3.0, 4.0], atol=1e-15)
    # Logits 0, -1: x = (1, 0.5), e = -2, codes 4 and 2: exact.
    np.testing.assert_allclose(_keys([0.0, -1.0], v, [(0, 2)]), (v[0] + 0.5 * v[1]) / 1.5, atol=1e-15)
    # x = (1, 0.3): 0.3 * 4 = 1.2 rounds to 1.0, so P = (1, 0.25), and the row sum is
    # that of the rounded values (1.25, not 1.3).
    np.testing.assert_allclose(_keys([0.0, math.log2(0.3)], v, [(0, 2)]),
                               (v[0] + 0.25 * v[1]) / 1.25, atol=1e-15)
    # x = (1, 0.09) in one MX block: 0.36 -> 0.5, P = 0.125; in two blocks the
    # second has its own scale 2^-6: 5.76 -> 6, P = 0.09375.
    np.testing.assert_allclose(_keys([0.0, math.log2(0.09)], v, [(0, 2)]),
                               (v[0] + 0.125 * v[1]) / 1.125, atol=1e-15)
    np.testing.assert_allclose(_keys([0.0, math.log2(0.09)], v, [(0, 1), (1, 2)]),
                               (v[0] + 0.09375 * v[1]) / 1.09375, atol=1e-15)
    # The reference is ceil(max) = 1, not the maximum 0.3: x = (2^-0.7, 2^-1), e = -3,
    # 4.92 -> 4 and 4 -> 4: equal P. With the maximum as reference x = (1, 0.81),
    # e = -2, 4 and 3.25 -> 3: P = (1, 0.75).
    np.testing.assert_allclose(_keys([0.3, 0.0], v, [(0, 2)]), (v[0] + v[1]) / 2, atol=1e-15)
    # Any integer shift of the logits leaves the output unchanged.
    rng = np.random.default_rng(16)
    ts = rng.uniform(-6, 0, 40)
    vv = rng.standard_normal((40, 3))
    base = _keys(ts, vv, [(0, 32), (32, 40)])
    for s in (-3, 1, 7):
        np.testing.assert_allclose(_keys(ts + s, vv, [(0, 32), (32, 40)]), base, atol=1e-14)
    # No keys: zeros.
    assert np.all(attention_block_mxp(np.ones((2, 3)), np.zeros((0, 3)), np.zeros((0, 4)), 1.0, []) == 0)


def test_mxp_within_rounding_bound_of_exact_softmax():
    # |O_q - O| = |sum (P~ - P)(v - O)| / sum P~ <= max|v - O| * sum bound(P) / sum P~
    rng = np.random.default_rng(17)
    q = rng.standard_normal((16, 32))
    k = rng.standard_normal((300, 32))
    v = rng.standard_normal((300, 8))
    scale = 1 / math.sqrt(32)
    groups = [(a, min(a + 32, 300)) for a in range(0, 300, 32)]
    exact = attention_block(q, k, v, scale)
    quant = attention_block_mxp(q, k, v, scale, groups)
    t = scale / math.log(2.0) * (q @ k.T)
    x = np.exp2(t - np.ceil(t.max(axis=1, keepdims=True)))
    pq = mx_round_groups(x, groups)
    b = np.zeros_like(x)
    for a, c in groups:
        e = mx_scale_exponent(x[:, a:c].max(axis=1)).astype(float)[:, None]
        b[:, a:c] = _err_bound(x[:, a:c], e)
    assert np.all(np.abs(pq - x) <= b * (1 + 1e-12))
    spread = np.abs(v[None, :, :] - exact[:, None, :]).max(axis=1)
    bound = spread * (b.sum(axis=1) / pq.sum(axis=1))[:, None]
    assert np.all(np.abs(quant - exact) <= bound * (1 + 1e-12))
    assert np.abs(quant - exact).max() > 0


def test_listed_groups_follow_block_quarters():
    g = Geometry(512, (62, 24, 42), False, 0.8)               # last tail block: 32 rows
    p = plan(g)
    ids = [0, p.n_blocks - 1, 5]
    groups = listed_groups(p, ids)
    sizes = [b - a for a, b in groups]
    n_last = p.blocks[-1][1]
    assert n_last % 128 != 0
    assert sizes == [32] * 4 + [min(32, n_last - a) for a in range(0, n_last, 32)] + [32] * 4
    assert groups[0][0] == 0 and all(a == b for (_, a), (b, _) in zip(groups, groups[1:]))


def test_mxfp4_pipeline_wiring():
    g = Geometry(128, (9, 16, 32), True, 0.8)
    rng = np.random.default_rng(18)
    q, k, v = (rng.standard_normal((1, 2, g.seq_len, 64)).astype(np.float32) for _ in range(3))
    r = oracle.run(q, k, v, g, precision="mxfp4")
    b = oracle.run(q, k, v, g, precision="bf16")
    assert np.array_equal(r["select_idx"], b["select_idx"])      # selection on unquantised Q/K
    p = r["plan"]
    assert r["q4"].shape == (1, 2, g.seq_len, 64) and r["q_exp"].shape == (1, 2, g.seq_len, 2)
    assert r["v_exp"].shape == (1, 2, p.n_blocks, 4, 64)
    qd = dequantize_rows_mx(r["q4"], r["q_exp"])
    kd = dequantize_rows_mx(r["k4"], r["k_exp"])
    vd = dequantize_v_mx(r["v4"], r["v_exp"], p)
    ref = oracle.sparse_attention(qd, kd, vd, p, r["select_idx"], r["select_num"], r["scale"],
                                  quantize_p="mxfp4")
    np.testing.assert_allclose(r["out_p"], ref, rtol=0, atol=1e-13)
    # MXFP4 is coarse (one mantissa bit): close to bf16 on average, not element-wise.
    err = np.abs(r["out"] - b["out"])
    assert err.mean() < 0.35 * np.abs(b["out"]).mean() and err.max() < 0.2
    with pytest.raises(ValueError):
        oracle.sparse_attention(qd, kd, vd, p, r["select_idx"], r["select_num"], 1.0, quantize_p="fp4")
