"""Pins of the oracle's attention step and of the whole oracle pipeline.

Pins: sparsity 0 equals dense attention computed by an independent library
routine (torch's CPU scaled_dot_product_attention); the natural-order dense
attention under a boolean mask expanded from selectIdx equals the oracle;
closed forms (V constant => O constant; Q = 0 => O = plain mean of V over the
listed rows, which catches short-block masking); GQA equals MHA with K/V
repeated; TND equals BNSD; an empty list gives zeros.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.geometry import Geometry, plan, permutation


def _sdpa(q, k, v, scale, mask=None):
    t = [torch.from_numpy(np.asarray(a, dtype=np.float64)) for a in (q, k, v)]
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        t[0], t[1], t[2], attn_mask=m, scale=scale).numpy()


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("P,grid,f0", [(128, (9, 16, 32), True), (200, (5, 16, 24), False),
                                        (77, (6, 13, 21), True)])
def test_sparsity_zero_is_dense_attention(P, grid, f0):
    g = Geometry(P, grid, f0, 0.0)
    S = g.seq_len
    q, k, v = _rand((1, 2, S, 16), 1), _rand((1, 2, S, 16), 2), _rand((1, 2, S, 16), 3)
    res = oracle.run(q, k, v, g, scale=0.3)
    assert res["plan"].fallback
    np.testing.assert_allclose(res["out"], _sdpa(q, k, v, 0.3), rtol=0, atol=1e-12)


def _natural_mask(g, sel_idx, sel_num, n):
    """Boolean [S, S] mask in natural order: query row may see key row."""
    p = plan(g)
    pi = permutation(g)
    S = g.seq_len
    mask = np.zeros((S, S), dtype=bool)
    for q in range(p.n_blocks):
        qr0, qn = p.blocks[q]
        qrows = pi[qr0:qr0 + qn]
        for j in sel_idx[q, n, :sel_num[q, n]]:
            kr0, kn = p.blocks[j]
            mask[np.ix_(qrows, pi[kr0:kr0 + kn])] = True
    return mask


@pytest.mark.parametrize("P,grid,f0,s", [(128, (9, 16, 32), True, 0.8),
                                          (100, (5, 16, 26), False, 0.5),
                                          (40, (7, 9, 17), True, 0.7)])
def test_masked_dense_attention_matches(P, grid, f0, s):
    g = Geometry(P, grid, f0, s, min_sparse_blocks=1)
    S = g.seq_len
    N = 2
    q, k, v = _rand((1, N, S, 16), 4), _rand((1, N, S, 16), 5), _rand((1, N, S, 16), 6)
    res = oracle.run(q, k, v, g, scale=0.25)
    p = res["plan"]
    assert not p.fallback and p.topk < p.n_sparse
    for n in range(N):
        mask = _natural_mask(g, res["select_idx"], res["select_num"], n)
        want = _sdpa(q[0, n], k[0, n], v[0, n], 0.25, mask)
        np.testing.assert_allclose(res["out"][0, n], want, rtol=0, atol=1e-12)


def test_constant_v_gives_constant_output():
    g = Geometry(512, (6, 24, 42), False, 0.8, min_sparse_blocks=1)  # unaligned w -> short tail block
    S = g.seq_len
    q, k = _rand((1, 1, S, 8), 7), _rand((1, 1, S, 8), 8)
    v = np.full((1, 1, S, 8), -1.25)
    out = oracle.run(q, k, v, g)["out"]
    np.testing.assert_allclose(out, -1.25, rtol=0, atol=1e-13)


def test_zero_q_gives_mean_of_listed_rows():
    g = Geometry(512, (6, 24, 42), False, 0.8, min_sparse_blocks=1)
    p = plan(g)
    assert p.blocks[-1][1] < 128  # a short tail block is present
    S = g.seq_len
    q = np.zeros((1, 1, S, 8))
    k, v = _rand((1, 1, S, 8), 9), _rand((1, 1, S, 8), 10)
    res = oracle.run(q, k, v, g)
    vp = res["vp"][0, 0]
    for qb in range(p.n_blocks):
        ids = res["select_idx"][qb, 0, :res["select_num"][qb, 0]]
        rows = np.concatenate([np.arange(p.blocks[j][0], p.blocks[j][0] + p.blocks[j][1])
                               for j in ids])
        r0, m = p.blocks[qb]
        np.testing.assert_allclose(res["out_p"][0, 0, r0:r0 + m],
                                   np.broadcast_to(vp[rows].mean(axis=0), (m, 8)), atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    g = Geometry(128, (9, 16, 32), True, 0.8)
    S = g.seq_len
    q = _rand((1, 4, S, 16), 11)
    k, v = _rand((1, 2, S, 16), 12), _rand((1, 2, S, 16), 13)
    a = oracle.run(q, k, v, g)
    b = oracle.run(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), g)
    assert np.array_equal(a["select_idx"], b["select_idx"])
    np.testing.assert_allclose(a["out"], b["out"], rtol=0, atol=1e-13)


def test_tnd_equals_bnsd_batch2():
    g = Geometry(128, (9, 16, 32), True, 0.8)
    S = g.seq_len
    q, k, v = _rand((2, 2, S, 8), 14), _rand((2, 2, S, 8), 15), _rand((2, 2, S, 8), 16)
    a = oracle.run(q, k, v, g, batch=2)

    def tnd(x):
        return x.transpose(0, 2, 1, 3).reshape(2 * S, x.shape[1], x.shape[3])
    b = oracle.run(tnd(q), tnd(k), tnd(v), g, layout="TND", batch=2)
    assert np.array_equal(a["select_idx"], b["select_idx"])
    np.testing.assert_allclose(tnd(a["out"]), b["out"], rtol=0, atol=1e-13)
    # The two batch items are independent: running item 1 alone gives the same rows.
    c = oracle.run(q[1:], k[1:], v[1:], g)
    np.testing.assert_allclose(c["out"][0], a["out"][1], rtol=0, atol=1e-13)


def test_empty_list_gives_zero_rows():
    # No prefix, no first frame, aligned grid, sparsity 1: sparse rows keep nothing.
    g = Geometry(0, (4, 16, 16), False, 1.0, min_sparse_blocks=1)
    S = g.seq_len
    q, k, v = _rand((1, 1, S, 8), 17), _rand((1, 1, S, 8), 18), _rand((1, 1, S, 8), 19)
    res = oracle.run(q, k, v, g)
    assert np.all(res["select_num"] == 0)
    assert np.all(res["out"] == 0)
