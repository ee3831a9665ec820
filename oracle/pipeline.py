"""The whole path, step by step, in the order the pages give it.

TEST INFRASTRUCTURE (see the package docstring).

1. arrange the tokens (permutation pi, ``geometry.py``);
2. pool the sparse blocks of Q and K (``select.py``);
3. score and keep the top-k key blocks per sparse query block (``select.py``);
4. exact softmax attention over the listed blocks (``attention.py``),
   with Q/K replaced by their fp8 E4M3 dequantised values in "mix" and "fp8"
   precision, V by its power-of-two-scaled E4M3 values and P by E4M3
   exponentials in "fp8" (``fp8.py``, ``attention.py``); in "mxfp4" every
   operand and P in MXFP4 with UOS scales (``mxfp4.py``, ``attention.py``);
   selection always uses the unquantised Q/K;
5. undo the arrangement.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import sparse_attention
from .fp8 import e4m3_decode, quantize_blocks, quantize_blocks_pow2
from .mxfp4 import dequantize_rows_mx, dequantize_v_mx, quantize_rows_mx, quantize_v_mx
from .geometry import Geometry, permutation, permute_rows, plan, unpermute_rows
from .select import block_scores, pool_blocks, select_lists


def _expand_block_scale(sigma: np.ndarray, p, S: int) -> np.ndarray:
    """Per-row copy of a per-block scale: ``[B, N, n_blocks] -> [B, N, S, 1]``."""
    rows = np.empty((sigma.shape[0], sigma.shape[1], S, 1), dtype=np.float64)
    for j, (r0, n) in enumerate(p.blocks):
        rows[:, :, r0:r0 + n, 0] = sigma[:, :, j:j + 1]
    return rows


def run(q, k, v, g: Geometry, scale: float | None = None, precision: str = "bf16",
        layout: str = "BNSD", batch: int = 1, query_blocks=None, select=None) -> dict:
    """Run the path on float inputs (bf16 values widened to float32/float64).

    ``q``: BNSD ``[B, N1, S, D]`` or TND ``[B*S, N1, D]``; ``k``, ``v`` likewise
    with N2 heads. ``select``: optional ``(select_idx, select_num)`` to use
    instead of the oracle's own selection (to check the attention step alone).
    ``query_blocks``: optional subset of ``(b, q, n)`` for the attention step.
    """
    if layout == "TND":
        def to_bnsd(x):
            t, n, d = x.shape
            return x.reshape(batch, t // batch, n, d).transpose(0, 2, 1, 3)
        q, k, v = to_bnsd(q), to_bnsd(k), to_bnsd(v)
    elif layout != "BNSD":
        raise ValueError(f"layout must be BNSD or TND, got {layout!r}")
    B, N1, S, D = q.shape
    if S != g.seq_len:
        raise ValueError(f"sequence length {S} does not match the geometry ({g.seq_len})")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    p = plan(g)
    pi = permutation(g)
    qp, kp, vp = (permute_rows(x, pi) for x in (q, k, v))
    res = dict(plan=p, pi=pi, qp=qp, kp=kp, vp=vp, scale=scale)
    if p.fallback:
        res.update(q_pool=None, k_pool=None, scores=None)
        sel = select_lists(p, B, N1)
    else:
        res["q_pool"] = pool_blocks(qp, p)
        res["k_pool"] = pool_blocks(kp, p)
        res["scores"] = block_scores(res["q_pool"], res["k_pool"], scale)
        sel = select_lists(p, B, N1, res["scores"])
    res["select_idx"], res["select_num"] = sel
    if select is not None:
        sel = select
    q_att, k_att, v_att = qp, kp, vp
    if precision in ("mix", "fp8"):
        q8, sq = quantize_blocks(qp, p)
        k8, sk = quantize_blocks(kp, p)
        res.update(q8=q8, k8=k8, q_scale=sq, k_scale=sk)
        q_att = e4m3_decode(q8) * _expand_block_scale(sq, p, S)
        k_att = e4m3_decode(k8) * _expand_block_scale(sk, p, S)
        if precision == "fp8":
            v8, sv = quantize_blocks_pow2(vp, p)
            res.update(v8=v8, v_scale=sv)
            v_att = e4m3_decode(v8) * _expand_block_scale(sv, p, S)
    elif precision == "mxfp4":
        q4, eq = quantize_rows_mx(qp)
        k4, ek = quantize_rows_mx(kp)
        v4, ev = quantize_v_mx(vp, p)
        res.update(q4=q4, k4=k4, v4=v4, q_exp=eq, k_exp=ek, v_exp=ev)
        q_att = dequantize_rows_mx(q4, eq)
        k_att = dequantize_rows_mx(k4, ek)
        v_att = dequantize_v_mx(v4, ev, p)
    elif precision != "bf16":
        raise ValueError(f"precision must be bf16, mix, fp8 or mxfp4, got {precision!r}")
    qmode = {"fp8": "fp8", "mxfp4": "mxfp4"}.get(precision, False)
    out_p = sparse_attention(q_att, k_att, v_att, p, sel[0], sel[1], scale, query_blocks,
                             quantize_p=qmode)
    res["out_p"] = out_p
    out = unpermute_rows(out_p, pi)
    if layout == "TND":
        out = out.transpose(0, 2, 1, 3).reshape(B * S, N1, D)
    res["out"] = out
    return res
