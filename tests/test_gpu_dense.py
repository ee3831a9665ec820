"""GPU parity of the dense path (rf_dense_attn through dense_attention).

The reference is textbook full attention over every key row, in the caller's
natural order, in float64 (oracle.attention_block per batch item and head):
full attention does not depend on the arrangement. The dense entry point must
also equal rf_sparse_attn with every block listed in order bit for bit (the
same kernel walking the same blocks), and the schedule front end must route
dense steps and layers to it.
"""
import numpy as np
import pytest

import oracle
from synth import WORKLOADS, Workload, make_qkv, to_tnd, from_tnd

from gpu_harness import (BF16_TOL, MIX_TOL, assert_close,
                         assert_within, fp8_bound_permuted, in_output_layout, mx_param, f32, log,
                         to_dev, to_host_u16)

pytestmark = pytest.mark.gpu


def _custom(name, batch, hq, hkv, d, prefix, grid, f0, s, precision="bf16"):
    return Workload(name, batch, hq, hkv, d, prefix, grid, f0, s, precision, True, 7)


CASES = {
    "tiny": (WORKLOADS["tiny"], "BNSD"),
    "tiny_mix": (WORKLOADS["tiny"].with_(precision="mix"), "BNSD"),
    "tiny_fp8": (WORKLOADS["tiny"].with_(precision="fp8"), "BNSD"),
    "ragged_gqa_fp8": (_custom("ragged_gqa", 1, 4, 2, 128, 200, (10, 17, 34), True, 0.8, "fp8"),
                       "BNSD"),
    "tiny_mxfp4": (WORKLOADS["tiny"].with_(precision="mxfp4"), "BNSD"),
    "ragged_gqa_mxfp4": (_custom("ragged_gqa", 1, 4, 2, 128, 200, (10, 17, 34), True, 0.8,
                                 "mxfp4"), "BNSD"),
    "tiny_tnd_b2": (WORKLOADS["tiny"].with_(batch=2), "TND"),
    "ragged_gqa": (_custom("ragged_gqa", 1, 4, 2, 128, 200, (10, 17, 34), True, 0.8), "BNSD"),
    "minimax_small": (_custom("minimax_small", 1, 2, 2, 128, 512, (6, 24, 42), False, 0.8),
                      "BNSD"),
    # geometry fallback (31 sparse blocks, below 32): identity arrangement, D=64
    "fallback_31": (_custom("fallback_31", 1, 2, 2, 64, 128, (3, 8, 248), True, 0.8), "BNSD"),
}


def _full_attention(q, k, v, scale):
    """[B, N1, S, D] float64 full attention, kv head n // G."""
    B, N1, S, D = q.shape
    G = N1 // k.shape[1]
    out = np.zeros((B, N1, S, D))
    for b in range(B):
        for n in range(N1):
            out[b, n] = oracle.attention_block(q[b, n], k[b, n // G], v[b, n // G], scale)
    return out


@pytest.mark.parametrize("name", [mx_param(n) for n in sorted(CASES)])
def test_dense_path_equals_full_attention(name):
    import torch
    import block_sparse_video_rf_amd as rf
    w, layout = CASES[name]
    desc = rf.Desc.from_workload(w, layout=layout)
    q, k, v = make_qkv(w)
    log(f"[dense {name}] S={w.seq_len} N={w.heads_q}/{w.heads_kv} D={w.head_dim} {w.precision} "
        f"{layout}")
    qi, ki, vi = (to_tnd(x) for x in (q, k, v)) if layout == "TND" else (q, k, v)
    out, bufs = rf.dense_attention(to_dev(qi), to_dev(ki), to_dev(vi), desc)
    torch.cuda.synchronize()
    assert bufs.select_idx is None  # the dense path builds no lists
    got = to_host_u16(out)
    if layout == "TND":
        got = from_tnd(got, w.batch)
    if w.precision == "mxfp4":
        # MXFP4 groups V and P by the quarters of the arranged blocks, so the
        # reference is the oracle's mxfp4 attention with every block listed
        # in that arrangement (the same quantised operands).
        from gpu_harness import geometry_of
        from oracle.geometry import plan
        p = plan(geometry_of(desc))
        nB = p.n_blocks
        idx = np.tile(np.arange(nB, dtype=np.int32), (w.batch * nB, w.heads_q, 1))
        num = np.full((w.batch * nB, w.heads_q), nB, dtype=np.int32)
        ores = oracle.run(f32(q), f32(k), f32(v), geometry_of(desc), precision="mxfp4",
                          select=(idx, num), batch=w.batch)
        kb = in_output_layout(fp8_bound_permuted(ores, (idx, num)), ores)
        assert_within(f32(got), ores["out"], kb, f"dense {name} vs mxfp4 reading")
        return
    ref = _full_attention(f32(q), f32(k), f32(v), 1.0 / np.sqrt(w.head_dim))
    if w.precision == "fp8":
        # The oracle's fp8 reading with every block listed (full attention on
        # the same E4M3 operands): the derived per-element bound against it, and
        # end to end no further from full attention than the reading is.
        from gpu_harness import geometry_of
        from oracle.geometry import plan
        p = plan(geometry_of(desc))
        nB = p.n_blocks
        sel = (np.tile(np.arange(nB, dtype=np.int32), (w.batch * nB, w.heads_q, 1)),
               np.full((w.batch * nB, w.heads_q), nB, dtype=np.int32))
        ores = oracle.run(f32(q), f32(k), f32(v), geometry_of(desc), precision="fp8",
                          select=sel, batch=w.batch)
        kb = in_output_layout(fp8_bound_permuted(ores, sel), ores)
        assert_within(f32(got), ores["out"], kb, f"dense {name} vs fp8 reading")
        assert_within(f32(got), ref, np.abs(ores["out"] - ref) + kb, f"dense {name} end to end")
        return
    tol = {"bf16": BF16_TOL, "mix": MIX_TOL}[w.precision]
    assert_close(f32(got), ref, tol, f"dense {name}")


@pytest.mark.parametrize("name", [mx_param(n) for n in ("ragged_gqa", "tiny_mix", "ragged_gqa_fp8",
                                                        "ragged_gqa_mxfp4")])
def test_dense_entry_point_equals_sparse_kernel_with_every_block(name):
    import torch
    import block_sparse_video_rf_amd as rf
    w, layout = CASES[name]
    desc = rf.Desc.from_workload(w, layout=layout)
    q, k, v = make_qkv(w)
    out, b = rf.attention(to_dev(q), to_dev(k), to_dev(v), desc)  # fills the permuted buffers
    nB = b.info.n_blocks
    rows = w.batch * nB
    idx = torch.arange(nB, dtype=torch.int32, device="cuda").repeat(rows, w.heads_q, 1)
    num = torch.full((rows, w.heads_q), nB, dtype=torch.int32, device="cuda")
    o_sparse = torch.empty_like(b.out_p)
    o_dense = torch.empty_like(b.out_p)
    rf.rf_sparse_attn(desc, b.qp, b.kp, b.vpt, b.q8, b.k8, b.q_scale, b.k_scale, b.v_scale, idx,
                      num, nB, o_sparse)
    rf.rf_dense_attn(desc, b.qp, b.kp, b.vpt, b.q8, b.k8, b.q_scale, b.k_scale, b.v_scale,
                     o_dense)
    torch.cuda.synchronize()
    assert torch.equal(o_sparse.view(torch.int16), o_dense.view(torch.int16))


def test_schedule_routes_dense_steps_and_layers():
    import torch
    import block_sparse_video_rf_amd as rf
    w = WORKLOADS["tiny"]
    desc = rf.Desc.from_workload(w)
    q, k, v = (to_dev(x) for x in make_qkv(w))
    sched = rf.DenseSchedule(start_step=1, end_step=1, skip_layers="3")
    sparse_out, _ = rf.attention(q, k, v, desc)
    dense_out, _ = rf.dense_attention(q, k, v, desc)
    bufs = None
    for step, layer, want in ((0, 0, False), (1, 0, True), (1, 3, False), (3, 1, False)):
        out, bufs, used_sparse = rf.scheduled_attention(q, k, v, desc, sched, step, 4, layer,
                                                        bufs=bufs)
        assert used_sparse == want
        torch.cuda.synchronize()
        ref = sparse_out if want else dense_out
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (step, layer)


def test_schedule_routes_geometry_fallback_dense():
    """31 sparse blocks (below the 32-block threshold): dense on every step."""
    import torch
    import block_sparse_video_rf_amd as rf
    w = _custom("fallback_31", 1, 2, 2, 64, 128, (3, 8, 248), True, 0.8)
    desc = rf.Desc.from_workload(w)
    q, k, v = (to_dev(x) for x in make_qkv(w))
    dense_out, _ = rf.dense_attention(q, k, v, desc)
    out, bufs, used_sparse = rf.scheduled_attention(q, k, v, desc, rf.DenseSchedule(), 2, 4, 5)
    torch.cuda.synchronize()
    assert bufs.info.dense_fallback == 1 and not used_sparse
    assert torch.equal(out.view(torch.int16), dense_out.view(torch.int16))


def test_dense_full_size_sampled_rows():
    """wan22 shapes, dense path: sampled query blocks against full attention."""
    import torch
    import block_sparse_video_rf_amd as rf
    w = WORKLOADS["wan22"]
    desc = rf.Desc.from_workload(w)
    q, k, v = make_qkv(w)
    log("[dense wan22] inputs ready")
    out, _ = rf.dense_attention(to_dev(q), to_dev(k), to_dev(v), desc)
    torch.cuda.synchronize()
    got = f32(to_host_u16(out))
    log("  gpu done")
    rng = np.random.default_rng(5)
    scale = 1.0 / np.sqrt(w.head_dim)
    for _ in range(6):
        n = int(rng.integers(w.heads_q))
        r0 = int(rng.integers(0, w.seq_len - 64))
        rows = slice(r0, r0 + 64)
        ref = oracle.attention_block(f32(q[0, n, rows]), f32(k[0, n]), f32(v[0, n]), scale)
        err = np.abs(got[0, n, rows].astype(np.float64) - ref)
        assert err.max() <= BF16_TOL[0] and err.mean() <= BF16_TOL[1], (n, r0, err.max())
    log("  6 sampled row blocks within tolerance")
