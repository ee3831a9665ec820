"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (the same four entry points, BNSD, one call each).

Everything the oracle can do quickly is compared in full: permuted Q/K and
block-transposed V (bit-exact), pooled means, the block scores in the
selection workspace, E4M3 codes and scales (bit-exact), selectIdx / selectNum
over every row (bit-exact up to near-ties). The Wan2.2 data in bf16, mix and
fp8 precision must select the same blocks (selection uses the unquantised
Q/K in every precision).

The attention output ("aclnnRainFusionAttention", Formula, over the listed
blocks) is compared through the inverse arrangement against the float64
oracle, spread over worker processes (tests/oracle_pool.py):
* bf16 and mix (wan22, minimax_h3, wan22_mix, gqa_long): every (query block,
  head) pair, the whole output;
* fp8 and mxfp4, whose per-element bounds cost far more than the oracle
  itself: every head at its first block, its last block, every 16th sparse
  block, and the query blocks of the last workgroup of each XCD's run in
  both dispatch phases (dense query blocks first, then sparse).

minimax_h3 also runs in the TND layout, which must reproduce the BNSD run bit
for bit (every intermediate buffer and the output).
"""
import numpy as np
import pytest

import oracle
from oracle.geometry import plan, permutation
from synth import WORKLOADS, make_qkv

from gpu_harness import (BF16_TOL, MIX_TOL, mx_v_scale_natural, unpack_e2m1, mx_param,
                         check_selection, expected_vpt, f32, geometry_of, log, run_gpu,
                         to_host_u16)
from oracle_pool import compare_pairs

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

XCDS = 8
_LISTS = {}   # selectIdx / selectNum of the Wan2.2 data, per precision


def _xcd_run_ends(p, batch, heads):
    """(b, q, n) of the last workgroup of each XCD's contiguous run, in both
    phases of the attention kernel's dispatch (its workgroup -> block map)."""
    n_dense = p.n_head + p.n_tail
    out = []
    for total, dense in ((batch * heads * n_dense, True), (batch * heads * p.n_sparse, False)):
        if total == 0:
            continue
        per, rem = divmod(total, XCDS)
        for x in range(XCDS):
            end = (x + 1) * per + min(x + 1, rem) - 1
            if end < 0 or end >= total:
                continue
            if dense:
                bn, qd = divmod(end, n_dense)
                q = qd if qd < p.n_head else qd + p.n_sparse
            else:
                bn, qs = divmod(end, p.n_sparse)
                q = p.n_head + qs
            out.append((bn // heads, q, bn % heads))
    return out


def _pairs(p, batch, heads, full):
    if full:
        return [(b, q, n) for b in range(batch) for q in range(p.n_blocks) for n in range(heads)]
    qs = {0, p.n_blocks - 1} | set(range(p.n_head, p.n_head + p.n_sparse, 16))
    picks = {(b, q, n) for b in range(batch) for q in qs for n in range(heads)}
    picks |= set(_xcd_run_ends(p, batch, heads))
    return sorted(picks)


def _dequant(codes, sigma, p, dtype=np.float64):
    d = np.empty(codes.shape, dtype=dtype)
    for j, (r0, n) in enumerate(p.blocks):
        d[:, :, r0:r0 + n] = oracle.e4m3_decode(codes[:, :, r0:r0 + n]) * sigma[:, :, j, None, None]
    return d


@pytest.mark.parametrize("name", [mx_param(n) for n in ("wan22", "minimax_h3", "wan22_mix",
                                                        "wan22_fp8", "wan22_mxfp4", "gqa_long")])
def test_full_size(name):
    import torch
    import block_sparse_video_rf_amd as rf
    w = WORKLOADS[name]
    desc = rf.Desc.from_workload(w)
    log(f"[full {name}] N={w.heads_q}/{w.heads_kv} S={w.seq_len} grid={w.grid} s={w.sparsity} "
        f"{w.precision}")
    q, k, v = make_qkv(w)
    log("  inputs ready")
    res = run_gpu(desc, q, k, v)
    bufs = res["bufs"]
    log("  gpu done")
    g = geometry_of(desc)
    p = plan(g)
    pi = permutation(g)
    qp_o, kp_o, vp_o = (oracle.permute_rows(x, pi) for x in (q, k, v))
    if bufs.qp is not None:
        assert np.array_equal(to_host_u16(bufs.qp), qp_o)
        assert np.array_equal(to_host_u16(bufs.kp), kp_o)
    if w.precision == "fp8":
        v8, sv = oracle.quantize_blocks_pow2(f32(vp_o), p)
        assert np.array_equal(bufs.vpt.cpu().numpy(), expected_vpt(v8, p, w.head_dim))
        assert np.array_equal(bufs.v_scale.cpu().numpy(), sv)
    elif w.precision == "mxfp4":
        v4, ev = oracle.quantize_v_mx(f32(vp_o), p)
        assert np.array_equal(unpack_e2m1(bufs.vpt.cpu().numpy()), expected_vpt(v4, p, w.head_dim))
        assert np.array_equal(mx_v_scale_natural(bufs.v_scale.cpu().numpy()),
                              (ev + 127).astype(np.uint8))
    else:
        assert np.array_equal(to_host_u16(bufs.vpt), expected_vpt(vp_o, p, w.head_dim))
    log("  permute bit-exact")
    qpool_o = oracle.pool_blocks(f32(qp_o), p)
    kpool_o = oracle.pool_blocks(f32(kp_o), p)
    assert np.abs(bufs.q_pool.cpu().numpy() - qpool_o).max() <= 2e-6
    assert np.abs(bufs.k_pool.cpu().numpy() - kpool_o).max() <= 2e-6
    log("  pools within 2e-6")
    scale = 1.0 / np.sqrt(w.head_dim)
    scores = oracle.block_scores(qpool_o, kpool_o, scale)
    # The block scores the selection ranked: the first piece of the workspace,
    # fp32 [B, N1, nS, nS], within 1e-5 of each row's largest magnitude.
    nS = p.n_sparse
    ws_scores = bufs.workspace[:w.batch * w.heads_q * nS * nS * 4].view(
        torch.float32).cpu().numpy().reshape(w.batch, w.heads_q, nS, nS)
    dev = np.abs(ws_scores - scores).max(axis=-1)
    rel = dev / np.abs(scores).max(axis=-1)
    log(f"  block scores: worst row deviation {rel.max():.2e} of the row's largest magnitude")
    assert rel.max() <= 1e-5
    gi = bufs.select_idx.cpu().numpy()
    gn = bufs.select_num.cpu().numpy()
    swaps = check_selection(p, w.batch, w.heads_q, gi, gn, scores)
    log(f"  selection exact ({swaps} near-tie rows)")
    if name.startswith("wan22"):
        _LISTS[name] = (gi, gn)
        if "wan22" in _LISTS and name != "wan22":
            assert np.array_equal(gi, _LISTS["wan22"][0]) and np.array_equal(gn, _LISTS["wan22"][1])
            log("  selectIdx / selectNum identical to the bf16 workload's")
    q_att, k_att = f32(qp_o), f32(kp_o)
    arrays = dict(q=q_att, k=k_att, v=f32(vp_o))
    if w.precision in ("mix", "fp8"):
        q8, sq = oracle.quantize_blocks(q_att, p)
        k8, sk = oracle.quantize_blocks(k_att, p)
        assert np.array_equal(bufs.q8.cpu().numpy(), q8)
        assert np.array_equal(bufs.k8.cpu().numpy(), k8)
        assert np.array_equal(bufs.q_scale.cpu().numpy(), sq)
        assert np.array_equal(bufs.k_scale.cpu().numpy(), sk)
        log("  fp8 codes and scales bit-exact")
        arrays.update(qd=_dequant(q8, sq, p), kd=_dequant(k8, sk, p))
        if w.precision == "fp8":
            arrays["vd"] = _dequant(v8, sv, p, np.float32)   # power-of-two scales: exact
    if w.precision == "mxfp4":
        q4, eq = oracle.quantize_rows_mx(q_att)
        k4, ek = oracle.quantize_rows_mx(k_att)
        arrays.update(qd=oracle.dequantize_rows_mx(q4, eq), kd=oracle.dequantize_rows_mx(k4, ek),
                      vd=oracle.dequantize_v_mx(v4, ev, p))
    # The GPU's output back in permuted order, so each pair is a block of rows.
    arrays["out"] = oracle.permute_rows(f32(to_host_u16(res["out"])), pi)
    full = w.precision in ("bf16", "mix")
    pairs = _pairs(p, w.batch, w.heads_q, full)
    log(f"  attention: {len(pairs)} (query block, head) pairs of {w.batch * p.n_blocks * w.heads_q}"
        f"{' (the whole output)' if full else ''}")
    mode = w.precision
    tol = MIX_TOL if mode == "mix" else BF16_TOL
    results = compare_pairs(arrays, p.blocks, pairs, (gi, gn), scale, w.heads_q // w.heads_kv,
                            mode, tol=tol, kernel_tol=BF16_TOL)
    bad = [r["pair"] for r in results if not r["ok"]]
    n = sum(r["n"] for r in results)
    worst = max(r["max"] for r in results)
    mean = sum(r["sum"] for r in results) / n
    msg = f"  end to end: {n} outputs, max-abs {worst:.3e}, mean-abs {mean:.3e}"
    if mode != "bf16":
        msg += (f"; against the {mode} reading max-abs {max(r['same_max'] for r in results):.3e}, "
                f"mean-abs {sum(r['same_sum'] for r in results) / n:.3e}")
    if mode in ("fp8", "mxfp4"):
        msg += f", worst err/bound {max(r['ratio'] for r in results):.3f}"
    log(msg)
    assert not bad, bad[:10]
    assert mean <= (MIX_TOL if mode == "mix" else BF16_TOL)[1] or mode in ("fp8", "mxfp4")


def test_full_size_tnd_equals_bnsd():
    """minimax_h3 in the TND layout (the caller's [B*S, N, D] rows): every
    intermediate buffer and the output, brought back to BNSD, bit-identical to
    the BNSD run, whose whole output the test above holds to the oracle (the
    layouts differ only in how rows are addressed)."""
    import block_sparse_video_rf_amd as rf
    from synth import from_tnd, to_tnd
    w = WORKLOADS["minimax_h3"]
    log(f"[full {w.name} TND] N={w.heads_q}/{w.heads_kv} S={w.seq_len} grid={w.grid}")
    q, k, v = make_qkv(w)
    a = run_gpu(rf.Desc.from_workload(w), q, k, v)
    t = run_gpu(rf.Desc.from_workload(w, layout="TND"), to_tnd(q), to_tnd(k), to_tnd(v))
    ba, bt = a["bufs"], t["bufs"]
    for name in ("qp", "kp", "vpt"):
        assert np.array_equal(to_host_u16(getattr(ba, name)), to_host_u16(getattr(bt, name))), name
    for name in ("q_pool", "k_pool", "select_idx", "select_num"):
        assert np.array_equal(getattr(ba, name).cpu().numpy(), getattr(bt, name).cpu().numpy()), name
    out_a = to_host_u16(a["out"])
    out_t = from_tnd(to_host_u16(t["out"]), w.batch)
    assert np.array_equal(out_a, out_t)
    log(f"  TND: permuted Q/K/V, pools, lists and the {out_a.size} outputs bit-identical to BNSD")
