"""Token arrangement: segments, block table and the permutation pi.

TEST INFRASTRUCTURE (see the package docstring).

What the pages fix, and the reading taken where they are silent:

* Video tokens arrive in (t, h, w) raster order after the prefix rows (text,
  conditions, audio). "RainFusion Attention", introduction: video is arranged
  in (t, h, w) order; prefix rows stay dense.
* The first latent frame can be split off as an always-dense sink
  ("RainFusion Attention", introduction: first-frame blocks remain dense;
  the RainFusion2.0 abstract, insight 3: first-frame sink). ``first_frame``
  says whether it is; it then holds H*W rows.
* The remaining frames are taken in pairs, and each pair is cut into 8x8
  spatial tiles, so one sparse block is a 2x8x8 = 128-token space-time box
  (xLLM pull request, commit summary: "frame-pairing" V2 rearrange; "RainFusion
  Attention", Geometry handling: 8x8-aligned grids; 128-token blocks in the
  introduction). Blocks are numbered (pair, tile row, tile column) and the
  tokens inside a block (dt, dh, dw), both in raster order (reading).
* Tokens that do not fit a box (rows h >= 8*floor(H/8), columns
  w >= 8*floor(W/8) of paired frames, and a last unpaired frame) are promoted
  to an always-kept video tail in their natural order; nothing is padded
  ("RainFusion Attention", Geometry handling: the MiniMax-H3 grid (62, 24, 42)
  gives 62,496 video rows, 2,976 promoted, 59,520 = 465 x 128 sparse).
* Permuted order: prefix, first frame, sparse blocks, promoted tail. The head
  segment (prefix + first frame) and the tail are cut into 128-row blocks with
  a short last block (ceiling division, "aclnnRainFusionAttention"
  constraints); the sparse segment is exactly ``n_sparse`` full blocks.
* Fallback to plain dense attention (identity arrangement, every block
  dense) when there is no grid, when sparsity is 0 ("RainFusion Attention",
  Configuration: 0 disables sparsity), or when the video has fewer than 32
  sparse blocks ("RainFusion Attention", introduction: video segments below
  32 blocks go to dense attention).
* Number of kept sparse key blocks per query block:
  ``k = n_sparse - floor(s * n_sparse + 1e-6)`` in float64 (Configuration:
  ``sparsity`` is the nominal dropped fraction of key blocks; the 1e-6 guards
  products such as 0.9 * 1440 against rounding below an integer).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

BLOCK = 128
TILE = (2, 8, 8)


@dataclass(frozen=True)
class Geometry:
    """Per-batch-item sequence geometry: ``seq_len = prefix_len + T*H*W``."""
    prefix_len: int
    grid: Optional[Tuple[int, int, int]]  # None: no video geometry
    first_frame: bool
    sparsity: float
    min_sparse_blocks: int = 32

    @property
    def video_len(self) -> int:
        return 0 if self.grid is None else self.grid[0] * self.grid[1] * self.grid[2]

    @property
    def seq_len(self) -> int:
        return self.prefix_len + self.video_len


@dataclass
class Plan:
    seq_len: int
    fallback: bool
    head_rows: int        # prefix + first frame (or the whole sequence on fallback)
    first_frame_rows: int
    sparse_rows: int
    promoted_rows: int
    n_head: int
    n_sparse: int
    n_tail: int
    topk: int
    blocks: List[Tuple[int, int]] = field(default_factory=list)  # (row0, length) by block id

    @property
    def n_blocks(self) -> int:
        return self.n_head + self.n_sparse + self.n_tail

    @property
    def n_dense_kv(self) -> int:
        return self.n_head + self.n_tail

    def is_sparse_block(self, j: int) -> bool:
        return self.n_head <= j < self.n_head + self.n_sparse


def num_kept(n_sparse: int, sparsity: float) -> int:
    """Sparse key blocks kept per sparse query block (see module docstring)."""
    return n_sparse - int(math.floor(float(sparsity) * n_sparse + 1e-6))


def _tile_counts(g: Geometry):
    T, H, W = g.grid
    f0 = 1 if g.first_frame else 0
    pairs = (T - f0) // 2
    return f0, pairs, H // 8, W // 8


def _cut(row0: int, rows: int) -> List[Tuple[int, int]]:
    out = []
    r = 0
    while r < rows:
        out.append((row0 + r, min(BLOCK, rows - r)))
        r += BLOCK
    return out


def plan(g: Geometry) -> Plan:
    S = g.seq_len
    n_sparse = 0
    if g.grid is not None:
        f0, pairs, th, tw = _tile_counts(g)
        n_sparse = pairs * th * tw
    fallback = (g.grid is None or g.sparsity == 0.0 or n_sparse < g.min_sparse_blocks)
    if fallback:
        blocks = _cut(0, S)
        return Plan(S, True, S, 0, 0, 0, len(blocks), 0, 0, 0, blocks)
    T, H, W = g.grid
    F = H * W if g.first_frame else 0
    head = g.prefix_len + F
    sparse = BLOCK * n_sparse
    promoted = g.video_len - F - sparse
    hb = _cut(0, head)
    sb = [(head + BLOCK * j, BLOCK) for j in range(n_sparse)]
    tb = _cut(head + sparse, promoted)
    return Plan(S, False, head, F, sparse, promoted, len(hb), n_sparse, len(tb),
                num_kept(n_sparse, g.sparsity), hb + sb + tb)


def permutation(g: Geometry) -> np.ndarray:
    """``pi[r]`` = natural row of the token at permuted position ``r`` (int64, length S)."""
    p = plan(g)
    if p.fallback:
        return np.arange(g.seq_len, dtype=np.int64)
    T, H, W = g.grid
    f0, pairs, _, _ = _tile_counts(g)
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    t, h, w = t.ravel(), h.ravel(), w.ravel()
    natural = g.prefix_len + (t * H + h) * W + w
    is_first = (t == 0) if f0 else np.zeros_like(t, dtype=bool)
    tt = t - f0
    in_pair = (tt >= 0) & (tt < 2 * pairs)
    is_sparse = in_pair & (h < 8 * (H // 8)) & (w < 8 * (W // 8))
    is_promoted = ~is_first & ~is_sparse
    # Sparse tokens ordered by (pair, tile row, tile col, dt, dh, dw): np.lexsort's last key is primary.
    m = is_sparse
    order = np.lexsort((w[m] % 8, h[m] % 8, tt[m] % 2, w[m] // 8, h[m] // 8, tt[m] // 2))
    return np.concatenate([
        np.arange(g.prefix_len),
        natural[is_first],            # raster order
        natural[m][order],
        natural[is_promoted],         # natural (increasing) order
    ]).astype(np.int64)


def permute_rows(x: np.ndarray, pi: np.ndarray, axis: int = -2) -> np.ndarray:
    """``xp[..., r, :] = x[..., pi[r], :]`` along the sequence axis."""
    return np.take(x, pi, axis=axis)


def unpermute_rows(xp: np.ndarray, pi: np.ndarray, axis: int = -2) -> np.ndarray:
    """Inverse of :func:`permute_rows`: ``x[..., pi[r], :] = xp[..., r, :]``."""
    inv = np.empty_like(pi)
    inv[pi] = np.arange(pi.size, dtype=pi.dtype)
    return np.take(xp, inv, axis=axis)


def block_rows(p: Plan, j: int) -> np.ndarray:
    """Permuted row indices of block ``j``."""
    r0, n = p.blocks[j]
    return np.arange(r0, r0 + n)
