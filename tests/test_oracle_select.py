"""Pins of the oracle's pooling, block scores, top-k and selection lists.

Pins: closed forms (affine input pools to the box centre), brute force in
plain Python (dot products, full sorts), invariants (min kept >= max dropped,
ascending lists, -1 padding), and special cases (planted block, sparsity 0/1).
"""
import numpy as np
import pytest

import oracle
from oracle.geometry import Geometry, plan, permutation, permute_rows


def _coords(g):
    """Natural-order (t, h, w) of every row; prefix rows get -1."""
    T, H, W = g.grid
    t = np.full(g.seq_len, -1)
    h = np.full(g.seq_len, -1)
    w = np.full(g.seq_len, -1)
    idx = np.arange(T * H * W)
    t[g.prefix_len:] = idx // (H * W)
    h[g.prefix_len:] = (idx // W) % H
    w[g.prefix_len:] = idx % W
    return t, h, w


@pytest.mark.parametrize("P,grid,f0", [(128, (9, 16, 32), True), (512, (62, 24, 42), False),
                                        (100, (7, 17, 26), True)])
def test_pool_of_affine_field_is_box_centre(P, grid, f0):
    g = Geometry(P, grid, f0, 0.8, min_sparse_blocks=1)
    p = plan(g)
    t, h, w = _coords(g)
    coef = np.array([[3.0, -2.0, 5.0, 1.0], [-1.0, 4.0, 2.0, -7.0]])  # two channels
    x = np.stack([c[0] * t + c[1] * h + c[2] * w + c[3] for c in coef], axis=-1)
    xp = permute_rows(x[None, None], permutation(g))
    pooled = oracle.pool_blocks(xp, p)[0, 0]
    tiles_h, tiles_w = grid[1] // 8, grid[2] // 8
    for j in range(p.n_sparse):
        pair, rem = divmod(j, tiles_h * tiles_w)
        ti, tj = divmod(rem, tiles_w)
        tc = (1 if f0 else 0) + 2 * pair + 0.5
        hc, wc = 8 * ti + 3.5, 8 * tj + 3.5
        want = coef[:, 0] * tc + coef[:, 1] * hc + coef[:, 2] * wc + coef[:, 3]
        assert np.array_equal(pooled[j], want)


def test_pool_of_constant_is_constant():
    g = Geometry(64, (5, 16, 16), True, 0.8, min_sparse_blocks=1)
    p = plan(g)
    xp = np.full((1, 2, g.seq_len, 4), 0.375)
    assert np.all(oracle.pool_blocks(xp, p) == 0.375)


def test_scores_brute_force_gqa():
    rng = np.random.default_rng(3)
    B, N1, N2, nS, D = 2, 4, 2, 5, 3
    qb = rng.standard_normal((B, N1, nS, D))
    kb = rng.standard_normal((B, N2, nS, D))
    sc = oracle.block_scores(qb, kb, 0.25)
    for b in range(B):
        for n in range(N1):
            for i in range(nS):
                for j in range(nS):
                    dot = 0.0
                    for d in range(D):
                        dot += qb[b, n, i, d] * kb[b, n // 2, j, d]
                    assert abs(sc[b, n, i, j] - 0.25 * dot) < 1e-12


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(5)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        k = int(rng.integers(0, n + 1))
        s = rng.integers(-3, 4, size=n).astype(np.float64)  # many ties
        got = oracle.topk_sparse(s, k)
        want = sorted(sorted(range(n), key=lambda j: (-s[j], j))[:k])
        assert list(got) == want
        if 0 < k < n:
            kept = set(got)
            assert min(s[j] for j in kept) >= max(s[j] for j in range(n) if j not in kept)


def _run_select(g, qp, kp, scale=0.125):
    p = plan(g)
    qb, kb = oracle.pool_blocks(qp, p), oracle.pool_blocks(kp, p)
    sc = oracle.block_scores(qb, kb, scale)
    return p, sc, oracle.select_lists(p, qp.shape[0], qp.shape[1], sc)


@pytest.mark.parametrize("P,grid,f0", [(200, (9, 16, 32), True), (100, (6, 13, 26), True)])
def test_lists_structure(P, grid, f0):
    g = Geometry(P, grid, f0, 0.8, min_sparse_blocks=1)
    rng = np.random.default_rng(11)
    B, N = 2, 3
    qp = rng.standard_normal((B, N, g.seq_len, 8))
    kp = rng.standard_normal((B, N, g.seq_len, 8))
    p, sc, (idx, num) = _run_select(g, qp, kp)
    nB = p.n_blocks
    assert p.n_tail > 0 or P == 200
    assert idx.shape == (B * nB, N, nB) and num.shape == (B * nB, N)
    for row in range(B * nB):
        b, q = divmod(row, nB)
        for n in range(N):
            m = num[row, n]
            lst = idx[row, n, :m]
            assert np.all(idx[row, n, m:] == -1)
            assert np.all(np.diff(lst) > 0) and lst.min() >= 0 and lst.max() < nB
            if p.is_sparse_block(q):
                assert m == p.n_dense_kv + p.topk
                dense = set(range(p.n_head)) | set(range(p.n_head + p.n_sparse, nB))
                assert dense <= set(lst)
                chosen = np.array(sorted(set(lst) - dense)) - p.n_head
                want = sorted(sorted(range(p.n_sparse),
                                     key=lambda j: (-sc[b, n, q - p.n_head, j], j))[:p.topk])
                assert list(chosen) == want
            else:
                assert m == nB and list(lst) == list(range(nB))


def test_planted_block_is_chosen_by_every_row():
    g = Geometry(128, (9, 16, 32), True, 0.9)
    p = plan(g)
    rng = np.random.default_rng(2)
    pi = permutation(g)
    c = np.linspace(0.5, 1.5, 16)                  # common query direction
    q = rng.standard_normal((1, 1, g.seq_len, 16)) + c
    k = rng.standard_normal((1, 1, g.seq_len, 16))
    qp, kp = permute_rows(q, pi), permute_rows(k, pi)
    # Key block j* gets a mean along c, so every query mean scores it highest.
    jstar = 17
    r0, n = p.blocks[p.n_head + jstar]
    kp[0, 0, r0:r0 + n] += 50.0 * c
    p, sc, (idx, num) = _run_select(g, qp, kp)
    for q_ in range(p.n_head, p.n_head + p.n_sparse):
        assert p.n_head + jstar in idx[q_, 0, :num[q_, 0]]


def test_sparsity_extremes():
    g0 = Geometry(128, (9, 16, 32), True, 0.0)
    p0 = plan(g0)
    idx, num = oracle.select_lists(p0, 1, 2)
    assert p0.fallback and np.all(num == p0.n_blocks)
    g1 = Geometry(128, (9, 16, 32), True, 1.0)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 2, g1.seq_len, 8))
    p1, _, (idx, num) = _run_select(g1, x, x)
    assert p1.topk == 0
    for q_ in range(p1.n_head, p1.n_head + p1.n_sparse):
        assert list(idx[q_, 0, :num[q_, 0]]) == list(range(p1.n_head))
    # A tiny sparsity keeps every block.
    gs = Geometry(128, (9, 16, 32), True, 0.01)
    ps, _, (idx, num) = _run_select(gs, x, x)
    assert ps.topk == ps.n_sparse and np.all(num == ps.n_blocks)
