"""Exact softmax attention restricted to the listed key blocks.

TEST INFRASTRUCTURE (see the package docstring).

"aclnnRainFusionAttention", Formula: the output is
``softmax(scale * Q K^T + mask) V`` where the sparse block size is
blockShapeX x blockShapeY and selectIdx says which key blocks each query block
sees. Here the blocks are 128 x 128 and no additive mask is used (the
arrangement does not pad; "RainFusion Attention", Geometry handling), so for
a query row r of block q and query head n the key rows are exactly the rows of
the blocks listed in ``select_idx[b*n_blocks + q, n, :select_num[...]]``;
a short block contributes only its real rows. A row whose list is empty gets
an all-zero output (reading: this only happens at sparsity 1 with no dense
blocks).

Float64 throughout: logits, the row maximum, exponentials, the row sum and
the weighted sum of V.

"fp8" precision ("RainFusion Attention", Configuration, names it without a
definition) also quantises the probabilities. Reading, from the MXAttention
abstract (catalyzex author page): the unnormalised softmax exponentials are
quantised before the row sum (pre-normalisation quantisation), so the
normalisation holds by construction; and quantised attention operands carry
power-of-two scales. The row of exponentials is therefore quantised exactly
like a V block of this precision (``fp8.py``: power-of-two scale, the
smallest one that fits the largest magnitude under 448):

* logits in log2 units ``t_c = scale * <q, k_c> / ln 2``, exponentials
  ``2**t_c`` (unnormalised; no reference subtracted);
* block scale ``2**e`` with ``e`` the smallest integer such that
  ``max_c 2**t_c <= 448 * 2**e``, i.e. ``e = ceil(max_c t_c - log2(448))``;
* ``P_c = e4m3(2**(t_c - e))`` (nearest, ties to even): the largest lies in
  (224, 448], the top of E4M3's range;
* ``O = sum_c P_c v_c / sum_c P_c`` - the row sum is the sum of the quantised
  values that multiply V.

A scale that put the row maximum exactly at the top of the range would in
general not be a power of two; the power-of-two scale is what the pages'
microscaling uses, and it is data-free (no calibration or search).

"mxfp4" precision ("RainFusion Attention", Wan2.2 T2V quantization, names it;
MXAttention, abstract, gives the pre-normalisation step). Reading, in the same
shape as "fp8":

* ``t_c`` as above, ``M = ceil(max_c t_c)``, ``x_c = 2**(t_c - M)`` in (0, 1];
* the row's keys fall into MX blocks of 32: the quarters of each listed
  128-row block (``mxfp4.py``); each block of ``x`` is quantised to MXFP4
  with its own UOS scale, giving ``P_c``;
* ``O = sum_c P_c v_c / sum_c P_c``.

Each MX block carries its own power-of-two scale, so multiplying ``x`` by
``2**k`` multiplies every ``P_c`` by exactly ``2**k``: any integer reference
gives the same output, and a one-pass kernel that rescales by powers of two
matches this definition (up to the clamp of the scale at 2**-127, far below
the largest P).
"""
from __future__ import annotations

import numpy as np

from .fp8 import E4M3_MAX, e4m3_round
from .geometry import Plan
from .mxfp4 import MX_BLOCK, mx_round_groups


def attention_block(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Dense softmax attention of query rows ``q [M, D]`` over key rows ``k, v [L, D]`` (float64)."""
    q = np.asarray(q, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    logits = scale * (q @ np.asarray(k, dtype=np.float64).T)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return (e @ np.asarray(v, dtype=np.float64)) / e.sum(axis=1, keepdims=True)


def fp8p_scale_exponent(t: np.ndarray) -> np.ndarray:
    """Exponent ``e`` of the power-of-two block scale of each row's
    exponentials ``2**t`` (``t [M, L]``): the smallest integer with
    ``2**max(t) <= 448 * 2**e``, i.e. ``ceil(max t - log2 448)`` (shape ``[M, 1]``)."""
    return np.ceil(t.max(axis=1, keepdims=True) - np.log2(E4M3_MAX))


def attention_block_fp8p(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Attention with E4M3 probabilities quantised before the row sum (float64).

    ``q [M, D]`` against ``k, v [L, D]`` (already dequantised operands)."""
    q = np.asarray(q, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    t = (scale / np.log(2.0)) * (q @ np.asarray(k, dtype=np.float64).T)
    pq = e4m3_round(np.exp2(t - fp8p_scale_exponent(t)))
    return (pq @ np.asarray(v, dtype=np.float64)) / pq.sum(axis=1, keepdims=True)


def attention_block_mxp(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                        groups) -> np.ndarray:
    """Attention with MXFP4 probabilities quantised before the row sum (float64).

    ``q [M, D]`` against ``k, v [L, D]`` (already dequantised operands);
    ``groups``: the MX blocks of P as ``(start, stop)`` key ranges covering
    [0, L)."""
    q = np.asarray(q, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    t = (scale / np.log(2.0)) * (q @ np.asarray(k, dtype=np.float64).T)
    ref = np.ceil(t.max(axis=1, keepdims=True))
    pq = mx_round_groups(np.exp2(t - ref), groups)
    return (pq @ np.asarray(v, dtype=np.float64)) / pq.sum(axis=1, keepdims=True)


def listed_groups(p: Plan, ids):
    """MX blocks of the listed keys: the quarters of each listed block's real
    rows, as ranges into the concatenation that ``listed_rows`` returns."""
    groups, off = [], 0
    for j in ids:
        n = p.blocks[j][1]
        for a in range(0, n, MX_BLOCK):
            groups.append((off + a, off + min(a + MX_BLOCK, n)))
        off += n
    return groups


def listed_rows(p: Plan, ids) -> np.ndarray:
    """Permuted row indices covered by the listed block ids, in list order."""
    parts = [np.arange(p.blocks[j][0], p.blocks[j][0] + p.blocks[j][1]) for j in ids]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def sparse_attention(qp, kp, vp, p: Plan, select_idx, select_num, scale: float,
                     query_blocks=None, quantize_p=False) -> np.ndarray:
    """Permuted-order attention output ``[B, N1, S, D]`` (float64).

    ``qp``: ``[B, N1, S, D]``; ``kp``, ``vp``: ``[B, N2, S, D]`` (permuted rows,
    any real dtype). ``query_blocks``: optional iterable of ``(b, q, n)`` to
    evaluate only those (query block, head) pairs; other rows stay zero.
    ``quantize_p``: False; True or "fp8" for E4M3 probabilities
    (``attention_block_fp8p``); "mxfp4" for MXFP4 probabilities
    (``attention_block_mxp``).
    """
    if quantize_p not in (False, True, "fp8", "mxfp4"):
        raise ValueError(f"quantize_p must be False, True, 'fp8' or 'mxfp4', got {quantize_p!r}")
    mx = quantize_p == "mxfp4"
    block = attention_block_fp8p if quantize_p in (True, "fp8") else attention_block
    B, N1, S, D = qp.shape
    G = N1 // kp.shape[1]
    nB = p.n_blocks
    out = np.zeros((B, N1, S, D), dtype=np.float64)
    todo = query_blocks if query_blocks is not None else (
        (b, q, n) for b in range(B) for q in range(nB) for n in range(N1))
    for b, q, n in todo:
        r0, m = p.blocks[q]
        row = b * nB + q
        ids = select_idx[row, n, :select_num[row, n]]
        rows = listed_rows(p, ids)
        args = (qp[b, n, r0:r0 + m], kp[b, n // G, rows], vp[b, n // G, rows], scale)
        out[b, n, r0:r0 + m] = (attention_block_mxp(*args, listed_groups(p, ids)) if mx
                                else block(*args))
    return out
