"""Pins of the oracle's arrangement (segments, block table, permutation).

Each check compares the oracle with something other than itself: the numbers
the pages print (tests/golden/geometry_facts.json), brute-force enumeration
of the token sets in plain Python loops, or invariants (bijection, roundtrip).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle.geometry import Geometry, plan, permutation
from synth import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "geometry_facts.json")
FACTS = json.load(open(GOLDEN))


def test_minimax_h3_counts_from_the_page():
    f = FACTS["minimax_h3_1344x768"]
    w, h = f["image"]
    # One latent token covers 32x32 pixels in this model family.
    assert (h // 32, w // 32) == tuple(f["grid"][1:])
    g = Geometry(512, tuple(f["grid"]), first_frame=False, sparsity=0.8)
    p = plan(g)
    assert g.video_len == f["video_rows"]
    assert p.promoted_rows == f["promoted_rows"]
    assert p.sparse_rows == f["sparse_rows"]
    assert p.n_sparse == f["sparse_blocks"]
    assert p.sparse_rows == p.n_sparse * f["block_rows"]
    # The page's count needs every frame paired: a first-frame sink would change it.
    p1 = plan(Geometry(512, tuple(f["grid"]), first_frame=True, sparsity=0.8))
    assert p1.n_sparse != f["sparse_blocks"]


@pytest.mark.parametrize("img", FACTS["aligned_grid_rule"]["aligned_images"])
def test_aligned_images_have_no_promoted_rows(img):
    px = FACTS["aligned_grid_rule"]["pixels_per_latent"]
    W, H = img[0] // px, img[1] // px
    for T, f0 in ((21, True), (20, False), (9, True)):
        p = plan(Geometry(64, (T, H, W), f0, 0.8, min_sparse_blocks=1))
        assert p.promoted_rows == 0


@pytest.mark.parametrize("img", FACTS["aligned_grid_rule"]["unaligned_images"])
def test_unaligned_images_promote_a_suffix(img):
    px = FACTS["aligned_grid_rule"]["pixels_per_latent"]
    W, H = img[0] // px, img[1] // px
    p = plan(Geometry(64, (21, H, W), True, 0.8, min_sparse_blocks=1))
    assert p.promoted_rows > 0


def test_dense_fallback_threshold():
    thr = FACTS["dense_fallback"]["min_sparse_blocks"]
    # (3, 8, 248) with a first frame: one frame pair, 1 x 31 tiles -> 31 blocks.
    below = plan(Geometry(128, (3, 8, 8 * (thr - 1)), True, 0.8))
    at = plan(Geometry(128, (3, 8, 8 * thr), True, 0.8))
    assert below.fallback and below.n_sparse == 0 and below.n_head == -(-below.seq_len // 128)
    assert not at.fallback and at.n_sparse == thr
    assert plan(Geometry(128, (3, 8, 8 * thr), True, FACTS["dense_fallback"]["dense_sparsity"])).fallback
    assert plan(Geometry(4096, None, False, 0.8)).fallback


def _brute_sets(P, T, H, W, f0):
    """Classify every video token with plain loops."""
    first, sparse, promoted = [], [], []
    pairs = (T - f0) // 2
    for t in range(T):
        for h in range(H):
            for w in range(W):
                nat = P + (t * H + h) * W + w
                if f0 and t == 0:
                    first.append(nat)
                elif f0 <= t < f0 + 2 * pairs and h < 8 * (H // 8) and w < 8 * (W // 8):
                    sparse.append(nat)
                else:
                    promoted.append(nat)
    return first, sparse, promoted


GEOMS = [(128, (9, 16, 32), True), (512, (62, 24, 42), False), (100, (6, 19, 13), True),
         (0, (4, 8, 8), False), (37, (5, 16, 24), False), (300, (8, 11, 17), True),
         (130, (2, 8, 16), False), (64, (7, 9, 9), True)]


@pytest.mark.parametrize("P,grid,f0", GEOMS)
def test_counts_match_brute_force(P, grid, f0):
    g = Geometry(P, grid, f0, 0.8, min_sparse_blocks=1)
    p = plan(g)
    first, sparse, promoted = _brute_sets(P, *grid, f0)
    assert p.first_frame_rows == len(first)
    assert p.sparse_rows == len(sparse) == 128 * p.n_sparse
    assert p.promoted_rows == len(promoted)
    assert p.head_rows == P + len(first)
    # Block table: head and tail cut with ceiling division, short last block.
    assert p.n_head == -(-(P + len(first)) // 128)
    assert p.n_tail == -(-len(promoted) // 128)
    rows = sum(n for _, n in p.blocks)
    assert rows == g.seq_len
    r = 0
    for r0, n in p.blocks:
        assert r0 == r and 1 <= n <= 128
        r += n


@pytest.mark.parametrize("P,grid,f0", GEOMS)
def test_permutation_structure(P, grid, f0):
    g = Geometry(P, grid, f0, 0.8, min_sparse_blocks=1)
    p = plan(g)
    pi = permutation(g)
    T, H, W = grid
    assert np.array_equal(np.sort(pi), np.arange(g.seq_len))          # bijection
    assert np.array_equal(pi[:p.head_rows], np.arange(p.head_rows))  # head keeps its order
    first, sparse, promoted = _brute_sets(P, T, H, W, f0)
    tail = pi[p.head_rows + p.sparse_rows:]
    assert list(tail) == sorted(promoted)                             # tail: natural order
    # Each sparse block is a 2x8x8 box visited in (dt, dh, dw) raster order, and the
    # boxes are visited in (pair, tile row, tile col) raster order.
    tiles_h, tiles_w = H // 8, W // 8
    for j in range(p.n_sparse):
        r0, n = p.blocks[p.n_head + j]
        pair, rem = divmod(j, tiles_h * tiles_w)
        ti, tj = divmod(rem, tiles_w)
        want = []
        for dt, dh, dw in itertools.product(range(2), range(8), range(8)):
            t, h, w = f0 + 2 * pair + dt, 8 * ti + dh, 8 * tj + dw
            want.append(P + (t * H + h) * W + w)
        assert list(pi[r0:r0 + n]) == want


@pytest.mark.parametrize("P,grid,f0", GEOMS[:4])
def test_roundtrip_is_identity(P, grid, f0):
    """Rearrange followed by its inverse gives the input back, bit for bit."""
    g = Geometry(P, grid, f0, 0.8, min_sparse_blocks=1)
    pi = permutation(g)
    x = np.random.default_rng(7).standard_normal((2, 3, g.seq_len, 8)).astype(np.float32)
    xp = oracle.permute_rows(x, pi)
    assert not np.array_equal(xp, x) or np.array_equal(pi, np.arange(g.seq_len))
    assert np.array_equal(oracle.unpermute_rows(xp, pi), x)


# The five workloads: counts stated in their descriptions (first-frame rows,
# sparse blocks, promoted rows, kept blocks at their sparsity).
WORKLOAD_COUNTS = {
    "tiny": dict(F=512, nS=32, U=0, n_head=5, n_tail=0, k=7),
    "wan22": dict(F=2560, nS=400, U=0, n_head=24, n_tail=0, k=80),
    "minimax_h3": dict(F=0, nS=465, U=2976, n_head=4, n_tail=24, k=93),
    "wan22_mix": dict(F=2560, nS=400, U=0, n_head=24, n_tail=0, k=80),
    "gqa_long": dict(F=6144, nS=1440, U=0, n_head=52, n_tail=0, k=144),
}


@pytest.mark.parametrize("name", sorted(WORKLOAD_COUNTS))
def test_workload_geometry(name):
    w = WORKLOADS[name]
    c = WORKLOAD_COUNTS[name]
    p = plan(Geometry(w.prefix_len, w.grid, w.first_frame, w.sparsity))
    assert not p.fallback
    assert (p.first_frame_rows, p.n_sparse, p.promoted_rows) == (c["F"], c["nS"], c["U"])
    assert (p.n_head, p.n_tail, p.topk) == (c["n_head"], c["n_tail"], c["k"])
    if name == "minimax_h3":
        assert p.blocks[-1][1] == 2976 - 23 * 128  # short last tail block (32 rows)


def test_kept_count_rounding():
    # Nominal sparsity is the dropped fraction; products that land on an
    # integer must not lose a block to floating-point rounding.
    assert oracle.num_kept(400, 0.8) == 80
    assert oracle.num_kept(1440, 0.9) == 144
    assert oracle.num_kept(32, 0.8) == 7
    assert oracle.num_kept(465, 0.8) == 93
    assert oracle.num_kept(10, 0.0) == 10
    assert oracle.num_kept(10, 1.0) == 0
    for n in range(1, 300):
        for s in (0.5, 0.6, 0.7, 0.75, 0.8, 0.9):
            exact = n - (n * round(s * 100)) // 100  # integer arithmetic
            assert oracle.num_kept(n, s) == exact
