"""The fp8 reading evaluated in one pass, as a streaming kernel must, against its definition.

The reading quantises P = 2^(t - M + 8) to E4M3, with t the logits in log2 units
and M the integer ceiling of the row maximum. It follows the pre-normalisation
idea of the MXAttention abstract: exponentials are quantised before the row sum.
A one-pass evaluation cannot know M in advance. It keeps a running integer
reference, raises it as blocks arrive, and rescales its sums by the power of two
between references. A power-of-two rescale commutes with E4M3 rounding of normal
values, so the one-pass result equals the definition while the P that matter are
normal. The offset 2^8 keeps them normal down to 14 binades below the maximum.

Here the one-pass evaluation runs in float64 on a small workload. It uses two key
halves with separate state, merged at the end. The test checks it against the
oracle's two-pass definition. It also checks that without the offset (largest P
at 1), the two evaluations disagree, which is why the reading takes 2^8.
"""
import math

import numpy as np

import oracle
from oracle.attention import attention_block_fp8p, listed_rows
from oracle.fp8 import e4m3_decode, e4m3_round
from oracle.geometry import Geometry, plan
from synth import WORKLOADS, bf16_to_f32, make_qkv


def _two_pass(Q, K, V, scale, off):
    t = (scale / math.log(2.0)) * (Q @ K.T)
    M = np.ceil(t.max(axis=1, keepdims=True))
    pq = e4m3_round(np.exp2(t - M + off))
    return (pq @ V) / pq.sum(axis=1, keepdims=True)


def _one_pass(Q, kd, vd, p, ids, scale, off):
    """Blocks in list order, 64-key halves with separate state, merged at the end."""
    states = []
    for kh in range(2):
        m_run = np.full(Q.shape[0], -np.inf)
        l = np.zeros(Q.shape[0])
        O = np.zeros((Q.shape[0], vd.shape[1]))
        for j in ids:
            r0, n = p.blocks[j]
            lo, hi = r0 + 64 * kh, min(r0 + 64 * kh + 64, r0 + n)
            if hi <= lo:
                continue
            t = (scale / math.log(2.0)) * (Q @ kd[lo:hi].T)
            mc = t.max(axis=1)
            if np.any(mc > m_run):
                m_new = np.maximum(m_run, np.ceil(mc))
                a = np.where(np.isinf(m_run), 0.0, np.exp2(m_run - m_new))
                O *= a[:, None]
                l *= a
                m_run = m_new
            pq = e4m3_round(np.exp2(t - m_run[:, None] + off))
            l += pq.sum(axis=1)
            O += pq @ vd[lo:hi]
        states.append((m_run, l, O))
    (m0, l0, O0), (m1, l1, O1) = states
    mm = np.maximum(m0, m1)
    a0 = np.where(np.isinf(m0), 0.0, np.exp2(m0 - mm))
    a1 = np.where(np.isinf(m1), 0.0, np.exp2(m1 - mm))
    return (O0 * a0[:, None] + O1 * a1[:, None]) / (l0 * a0 + l1 * a1)[:, None]


def _case():
    w = WORKLOADS["tiny"].with_(precision="fp8", head_dim=128)
    g = Geometry(w.prefix_len, w.grid, True, w.sparsity)
    q, k, v = make_qkv(w)
    res = oracle.run(bf16_to_f32(q), bf16_to_f32(k), bf16_to_f32(v), g, precision="fp8")
    p = plan(g)

    def deq(codes, sig):
        d = np.empty(codes.shape)
        for j, (r0, n) in enumerate(p.blocks):
            d[:, :, r0:r0 + n] = e4m3_decode(codes[:, :, r0:r0 + n]) * sig[:, :, j, None, None]
        return d
    return (w, p, res, deq(res["q8"], res["q_scale"]), deq(res["k8"], res["k_scale"]),
            deq(res["v8"], res["v_scale"]))


def test_one_pass_matches_definition_with_offset():
    w, p, res, qd, kd, vd = _case()
    scale = 1.0 / math.sqrt(w.head_dim)
    worst = 0.0
    for qb in range(p.n_blocks):
        for n in range(w.heads_q):
            ids = res["select_idx"][qb, n, :res["select_num"][qb, n]]
            r0, m = p.blocks[qb]
            Q = qd[0, n, r0:r0 + m]
            rows = listed_rows(p, ids)
            ref = attention_block_fp8p(Q, kd[0, n, rows], vd[0, n, rows], scale)
            assert np.allclose(ref, _two_pass(Q, kd[0, n, rows], vd[0, n, rows], scale, 8.0),
                               rtol=0, atol=1e-12)
            got = _one_pass(Q, kd[0, n], vd[0, n], p, ids, scale, 8.0)
            worst = max(worst, float(np.abs(got - ref).max()))
    assert worst <= 1e-5, worst


def test_without_offset_one_pass_departs_from_definition():
    w, p, res, qd, kd, vd = _case()
    scale = 1.0 / math.sqrt(w.head_dim)
    worst = 0.0
    for qb in range(p.n_blocks):
        for n in range(w.heads_q):
            ids = res["select_idx"][qb, n, :res["select_num"][qb, n]]
            r0, m = p.blocks[qb]
            Q = qd[0, n, r0:r0 + m]
            rows = listed_rows(p, ids)
            ref0 = _two_pass(Q, kd[0, n, rows], vd[0, n, rows], scale, 0.0)
            got0 = _one_pass(Q, kd[0, n], vd[0, n], p, ids, scale, 0.0)
            worst = max(worst, float(np.abs(got0 - ref0).max()))
    assert worst > 1e-3, worst
