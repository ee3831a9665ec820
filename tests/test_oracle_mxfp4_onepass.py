"""The kernel's one-pass evaluation of the mxfp4 reading, on the CPU, against
the oracle, and the derived per-element bound that the GPU tests use.

The reading (oracle/attention.py, ``attention_block_mxp``) quantises each
row's exponentials 2^(t - ref), ref the integer ceiling of the row maximum, per
MX block of 32 keys with the block's UOS scale. A streaming kernel keeps a
running integer reference instead, raised as blocks arrive, and takes each MX
block's scale from that block's own maximum: both shift the exponentials and
the scale by the same power of two, so in exact arithmetic the codes, and the
result, are the definition's. The checks:

* the one-pass evaluation in float64 equals the definition;
* with the GPU's arithmetic errors simulated at the sizes the bound assumes
  (logits within the matrix product's error model, exponentials within
  2^-20), codes flip next to E2M1 midpoints and scale boundaries, and the
  result stays within ``mx_kernel_bound``;
* plausible mistakes exceed that bound: one scale per row instead of per MX
  block, the 6.0 boundary of a plain amax/6 scale instead of 7.25,
  exponentials left unrounded, and the row sum of the unrounded values.
"""
import math

import numpy as np

import oracle
from oracle.attention import attention_block_mxp, listed_groups, listed_rows
from oracle.geometry import Geometry, plan
from oracle.mxfp4 import e2m1_decode, e2m1_encode, mx_scale_exponent
from synth import WORKLOADS, bf16_to_f32, make_qkv

from fp8_bounds import logit_error, mx_kernel_bound


def _uos(amax, qmax):
    """Smallest integer e with amax <= qmax * 2^e (amax > 0)."""
    e = np.ceil(np.log2(amax / qmax))
    e = np.where(qmax * np.exp2(e) < amax, e + 1, e)
    return np.where(qmax * np.exp2(e - 1) >= amax, e - 1, e)


def _one_pass(Q, kd, vd, p, ids, scale, noise=None, per_row_scale=False, qmax=7.25,
              round_p=True, sum_unrounded=False):
    """Blocks in list order; two 64-key halves with separate state (running
    integer reference m, sum l, output O), merged at the end; per MX block
    (32 keys of a half) the scale from the block's own maximum. ``noise``:
    (rng, logit error bound per listed key [M, L]) to perturb the logits and
    exponentials within the GPU's error model."""
    rows = listed_rows(p, ids)
    pos = {r: i for i, r in enumerate(rows)}
    rng, lerr = noise if noise is not None else (None, None)
    states = []
    for kh in range(2):
        m = np.full(Q.shape[0], -np.inf)
        l = np.zeros(Q.shape[0])
        O = np.zeros((Q.shape[0], vd.shape[1]))
        for j in ids:
            r0, n = p.blocks[j]
            lo, hi = r0 + 64 * kh, min(r0 + 64 * kh + 64, r0 + n)
            if hi <= lo:
                continue
            t = (scale / math.log(2.0)) * (Q @ kd[lo:hi].T)
            if rng is not None:
                cols = [pos[r] for r in range(lo, hi)]
                t = t + lerr[:, cols] * rng.uniform(-1.0, 1.0, t.shape)
            m_new = np.maximum(m, np.ceil(t.max(axis=1)))
            a = np.where(np.isinf(m), 0.0, np.exp2(m - m_new))
            O *= a[:, None]
            l *= a
            m = m_new
            for g0 in range(lo, hi, 32):
                g1 = min(g0 + 32, hi)
                tg = t[:, g0 - lo:g1 - lo]
                x = np.exp2(tg - m[:, None])
                if rng is not None:
                    x = x * (1.0 + 2.0 ** -20 * rng.uniform(-1.0, 1.0, x.shape))
                if per_row_scale:
                    amax = np.exp2(t.max(axis=1) - m)
                else:
                    amax = x.max(axis=1)
                e = _uos(amax, qmax)[:, None]
                pq = e2m1_decode(e2m1_encode(x / np.exp2(e))) * np.exp2(e) if round_p else x
                l += (x if sum_unrounded else pq).sum(axis=1)
                O += pq @ vd[g0:g1]
        states.append((m, l, O))
    (m0, l0, O0), (m1, l1, O1) = states
    mm = np.maximum(m0, m1)
    a0 = np.where(np.isinf(m0), 0.0, np.exp2(m0 - mm))
    a1 = np.where(np.isinf(m1), 0.0, np.exp2(m1 - mm))
    return (O0 * a0[:, None] + O1 * a1[:, None]) / (l0 * a0 + l1 * a1)[:, None]


def _case():
    w = WORKLOADS["tiny"].with_(precision="mxfp4", head_dim=128)
    g = Geometry(w.prefix_len, w.grid, True, w.sparsity)
    q, k, v = make_qkv(w)
    res = oracle.run(bf16_to_f32(q), bf16_to_f32(k), bf16_to_f32(v), g, precision="mxfp4")
    p = plan(g)
    qd = oracle.dequantize_rows_mx(res["q4"], res["q_exp"])
    kd = oracle.dequantize_rows_mx(res["k4"], res["k_exp"])
    vd = oracle.dequantize_v_mx(res["v4"], res["v_exp"], p)
    return w, p, res, qd, kd, vd


def _compare(heads=(0,), stride=1, noisy=False, **kw):
    """Worst |one pass - definition| and worst ratio to mx_kernel_bound."""
    w, p, res, qd, kd, vd = _case()
    scale = 1.0 / math.sqrt(w.head_dim)
    rng = np.random.default_rng(11)
    worst, ratio = 0.0, 0.0
    for qb in range(0, p.n_blocks, stride):
        for n in heads:
            ids = res["select_idx"][qb, n, :res["select_num"][qb, n]]
            r0, m = p.blocks[qb]
            Q = qd[0, n, r0:r0 + m]
            rows = listed_rows(p, ids)
            groups = listed_groups(p, ids)
            ref = attention_block_mxp(Q, kd[0, n, rows], vd[0, n, rows], scale, groups)
            noise = (rng, logit_error(Q, kd[0, n, rows], scale)) if noisy else None
            got = _one_pass(Q, kd[0, n], vd[0, n], p, ids, scale, noise=noise, **kw)
            err = np.abs(got - ref)
            worst = max(worst, float(err.max()))
            bound = mx_kernel_bound(Q, kd[0, n, rows], vd[0, n, rows], scale, groups)
            ratio = max(ratio, float((err / bound).max()))
    return worst, ratio


def test_one_pass_equals_definition():
    worst, ratio = _compare(heads=(0, 1))
    assert worst <= 1e-12 and ratio < 1e-3


def test_simulated_gpu_errors_within_derived_bound():
    """Logits and exponentials perturbed within the bound's error model: some
    codes flip (the result moves), and every element stays within the bound."""
    worst, ratio = _compare(heads=(0, 1), noisy=True)
    assert worst > 1e-4 and ratio < 1.0


def test_bound_catches_planted_mistakes():
    assert _compare(stride=3, per_row_scale=True)[1] > 1.0
    assert _compare(stride=3, qmax=6.0)[1] > 1.0
    assert _compare(stride=3, round_p=False)[1] > 1.0
    assert _compare(stride=3, sum_unrounded=True)[1] > 1.0


def test_scale_rule_matches_oracle():
    """The test's UOS helper is the oracle's rule (the kernel's is pinned on the
    host in test_host_mx.py)."""
    a = np.exp2(np.linspace(-20, 20, 4001)) * 7.25
    a = np.concatenate([a, np.nextafter(a, 0), np.nextafter(a, np.inf)])
    assert np.array_equal(_uos(a, 7.25).astype(np.int64), mx_scale_exponent(a))
