"""Block-mean pooling, block scores, top-k and the selectIdx / selectNum lists.

TEST INFRASTRUCTURE (see the package docstring).

* Pooling: the representative token of a sparse block is the mean of its 128
  permuted rows, for Q (every query head) and K (every KV head)
  ("RainFusion Attention", introduction: 128-token key blocks are pooled;
  RainFusion2.0 abstract, insight 1: block-wise mean values as representative
  tokens). Reading: Q is pooled the same way, since ranking is per query block.
* Score of query block i against key block j for query head n:
  ``scale * <qbar[n, i], kbar[n // G, j]>``. Reading: a plain scaled dot
  product of the means; a softmax over it would not change the ranking.
* Ranking: per sparse query block and query head, keep the ``k`` highest
  scores among the sparse key blocks ("RainFusion Attention", introduction:
  ranks pooled key blocks per query block and attends to the highest-scoring
  ones). Ties (reading): equal scores prefer the lower block id.
* Lists ("aclnnRainFusionAttention", Formula and constraints): selectIdx has
  shape ``[B*n_blocks, heads_q, max_kv]`` with the per-batch query blocks
  stacked batch-major, and invalid entries set to -1; selectNum has shape
  ``[B*n_blocks, heads_q]``. Reading: a sparse query block lists every dense
  block (head segment and promoted tail) plus its chosen sparse blocks, in
  increasing block id; a dense query block (head or tail segment) lists every
  block. ``max_kv = n_blocks``.

Everything is float64; the GQA kv head of query head n is ``n // G`` with
``G = heads_q / heads_kv`` (contiguous groups, reading of the garbled GQA
constraint on the operator page).
"""
from __future__ import annotations

import numpy as np

from .geometry import BLOCK, Plan, num_kept  # noqa: F401  (num_kept re-exported)


def pool_blocks(xp: np.ndarray, p: Plan) -> np.ndarray:
    """Means of the sparse blocks. ``xp``: permuted ``[B, N, S, D]`` -> ``[B, N, n_sparse, D]`` float64."""
    B, N, S, D = xp.shape
    out = np.zeros((B, N, p.n_sparse, D), dtype=np.float64)
    for j in range(p.n_sparse):
        r0, n = p.blocks[p.n_head + j]
        assert n == BLOCK
        out[:, :, j, :] = xp[:, :, r0:r0 + n, :].astype(np.float64).sum(axis=2) / n
    return out


def block_scores(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """``[B, N1, nS, D] x [B, N2, nS, D] -> [B, N1, nS, nS]`` scaled dot products (float64)."""
    B, N1 = qbar.shape[:2]
    G = N1 // kbar.shape[1]
    out = np.empty((B, N1, qbar.shape[2], kbar.shape[2]), dtype=np.float64)
    for b in range(B):
        for n in range(N1):
            out[b, n] = scale * (qbar[b, n].astype(np.float64) @ kbar[b, n // G].astype(np.float64).T)
    return out


def topk_sparse(scores_row: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k best sparse key blocks: higher score first, then lower index; sorted ascending."""
    idx = np.arange(scores_row.size)
    order = np.lexsort((idx, -scores_row))  # primary: -score; secondary: index
    return np.sort(order[:k])


def select_lists(p: Plan, batch: int, heads_q: int, scores=None):
    """Build ``(select_idx, select_num)`` (int32) from the plan and the block scores.

    ``scores``: ``[B, N1, nS, nS]`` or None when the plan is a dense fallback.
    """
    nB = p.n_blocks
    sel_idx = np.full((batch * nB, heads_q, nB), -1, dtype=np.int32)
    sel_num = np.zeros((batch * nB, heads_q), dtype=np.int32)
    all_blocks = np.arange(nB, dtype=np.int32)
    head_ids = np.arange(p.n_head, dtype=np.int32)
    tail_ids = np.arange(p.n_head + p.n_sparse, nB, dtype=np.int32)
    for b in range(batch):
        for q in range(nB):
            row = b * nB + q
            for n in range(heads_q):
                if p.is_sparse_block(q):
                    chosen = topk_sparse(scores[b, n, q - p.n_head], p.topk) + p.n_head
                    lst = np.concatenate([head_ids, chosen.astype(np.int32), tail_ids])
                else:
                    lst = all_blocks
                sel_idx[row, n, :lst.size] = lst
                sel_num[row, n] = lst.size
    return sel_idx, sel_num
