"""The kernel's one-pass evaluation of the fp8 reading, on the CPU, against the oracle.

This checks the kernel's algorithm, not the reading: the reading is fixed by
the pages alone (oracle/attention.py). It quantises each row's exponentials
2^t with the power-of-two block scale 2^e, e = ceil(max t - log2 448), as V
blocks are. A streaming kernel cannot know the row maximum in advance. It keeps
a running integer exponent, raises it as blocks arrive, and rescales its sums
by the power of two between exponents. A power-of-two rescale commutes with
E4M3 rounding of normal values, so the one-pass result equals the definition
while the P that matter are normal (the largest P lies in (224, 448], so P
stays normal down to about 15 binades below it).

Here the one-pass evaluation runs in float64 on a small workload, blocks in
list order, with two 64-key halves that keep separate state and merge at the
end, as the kernel does. On ordinary rows it matches the oracle's two-pass
definition; on rows whose exponent rises far mid-row, keys rounded as normal
values at an earlier exponent are subnormal at the final one, and the result
departs from the definition within the per-element bound that the GPU tests
use (tests/fp8_bounds.py). A one-pass evaluation that rescales by the running
maximum itself (a scale that is not a power of two), or that leaves P
unrounded, exceeds that bound.
"""
import math

import numpy as np

import oracle
from oracle.attention import attention_block_fp8p, listed_groups, listed_rows
from oracle.fp8 import e4m3_decode, e4m3_round
from oracle.geometry import Geometry, plan
from synth import WORKLOADS, bf16_to_f32, make_qkv

from fp8_bounds import kernel_bound

LOG2_448 = math.log2(448.0)


def _one_pass(Q, kd, vd, p, ids, scale, integer_exponent=True, round_p=True):
    """Blocks in list order, 64-key halves with separate state, merged at the end."""
    states = []
    for kh in range(2):
        e_run = np.full(Q.shape[0], -np.inf)
        l = np.zeros(Q.shape[0])
        O = np.zeros((Q.shape[0], vd.shape[1]))
        for j in ids:
            r0, n = p.blocks[j]
            lo, hi = r0 + 64 * kh, min(r0 + 64 * kh + 64, r0 + n)
            if hi <= lo:
                continue
            t = (scale / math.log(2.0)) * (Q @ kd[lo:hi].T)
            mt = t.max(axis=1) - LOG2_448
            if np.any(mt > e_run):
                e_new = np.maximum(e_run, np.ceil(mt) if integer_exponent else mt)
                a = np.where(np.isinf(e_run), 0.0, np.exp2(e_run - e_new))
                O *= a[:, None]
                l *= a
                e_run = e_new
            pq = np.exp2(t - e_run[:, None])
            if round_p:
                pq = e4m3_round(pq)
            l += pq.sum(axis=1)
            O += pq @ vd[lo:hi]
        states.append((e_run, l, O))
    (e0, l0, O0), (e1, l1, O1) = states
    ee = np.maximum(e0, e1)
    a0 = np.where(np.isinf(e0), 0.0, np.exp2(e0 - ee))
    a1 = np.where(np.isinf(e1), 0.0, np.exp2(e1 - ee))
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


def _compare(integer_exponent, key_scale=1.0, round_p=True):
    """Worst |one pass - definition|, and the worst ratio to the derived
    per-element bound of the GPU path (tests/fp8_bounds.py)."""
    w, p, res, qd, kd, vd = _case()
    kd = kd.copy()
    half = kd.shape[2] // 2
    kd[:, :, half:] *= key_scale          # later keys larger: the exponent must rise mid-row
    scale = 1.0 / math.sqrt(w.head_dim)
    worst, ratio = 0.0, 0.0
    for qb in range(p.n_blocks):
        for n in range(w.heads_q):
            ids = res["select_idx"][qb, n, :res["select_num"][qb, n]]
            r0, m = p.blocks[qb]
            Q = qd[0, n, r0:r0 + m]
            rows = listed_rows(p, ids)
            ref = attention_block_fp8p(Q, kd[0, n, rows], vd[0, n, rows], scale)
            got = _one_pass(Q, kd[0, n], vd[0, n], p, ids, scale, integer_exponent, round_p)
            err = np.abs(got - ref)
            worst = max(worst, float(err.max()))
            bound = kernel_bound(Q, kd[0, n, rows], vd[0, n, rows], scale, listed_groups(p, ids))
            ratio = max(ratio, float((err / bound).max()))
    return worst, ratio


def test_one_pass_matches_definition():
    worst, ratio = _compare(True)
    assert worst <= 1e-5 and ratio < 1.0


def test_one_pass_peaked_rows_within_derived_bound():
    """Later keys four times larger: the exponent rises mid-row, and keys
    rounded as normal values at the earlier exponent are subnormal at the
    final one. The one-pass result then departs from the definition (by
    about 4e-3 here), and stays within the derived per-element bound."""
    worst, ratio = _compare(True, key_scale=4.0)
    assert worst > 1e-4 and ratio < 1.0


def test_bound_catches_planted_mistakes():
    """A rescale by the running maximum itself (not a power of two), or
    exponentials left unrounded, exceed the bound."""
    assert _compare(False, key_scale=4.0)[1] > 1.0
    assert _compare(True, round_p=False)[1] > 1.0
