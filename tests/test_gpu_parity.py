"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small cases run every step in full: permuted copies (bit-exact), block
transposed V (bit-exact), pooled means, selectIdx/selectNum (bit-exact up to
documented near-ties), attention (oracle fed the GPU's own lists, and end to
end), the unpermuted output, and E4M3 codes/scales in mix precision. They span
several 128-row tiles and ragged tails: a prefix that is not a multiple of
128, unaligned grid height and width, an unpaired last frame, a short last
block, GQA, TND with batch 2, head_dim 64 and 128, and the degenerate cases
(dense fallback below 32 blocks, sparsity 0, sparsity 1 with empty lists).
"""
import numpy as np
import pytest

import oracle
from oracle.geometry import plan, permutation
from synth import WORKLOADS, Workload, make_qkv, to_tnd, from_tnd

from gpu_harness import (BF16_TOL, MIX_TOL, assert_close, assert_within,
                         check_selection, expected_vpt, f32, fp8_bound_permuted,
                         geometry_of, in_output_layout, log,
                         mx_param, mx_v_scale_natural, run_gpu, to_host_u16, unpack_e2m1,
                         case_desc, case_inputs, full_check)

pytestmark = pytest.mark.gpu


def _custom(name, batch, hq, hkv, d, prefix, grid, f0, s, precision="bf16", smooth=True, seed=7):
    return Workload(name, batch, hq, hkv, d, prefix, grid, f0, s, precision, smooth, seed)


SMALL = {
    "tiny": (WORKLOADS["tiny"], {}),
    "tiny_mix": (WORKLOADS["tiny"].with_(precision="mix"), {}),
    "tiny_tnd_b2": (WORKLOADS["tiny"].with_(batch=2), {"layout": "TND"}),
    # prefix not a multiple of 128, unaligned h and w, unpaired last frame, GQA 4/2, D=128
    "ragged_gqa": (_custom("ragged_gqa", 1, 4, 2, 128, 200, (10, 17, 34), True, 0.8), {}),
    "ragged_gqa_mix": (_custom("ragged_gqa", 1, 4, 2, 128, 200, (10, 17, 34), True, 0.8,
                               precision="mix"), {}),
    # MiniMax-like unaligned width, no first frame: a 32-row last tail block
    "minimax_small": (_custom("minimax_small", 1, 2, 2, 128, 512, (6, 24, 42), False, 0.8), {}),
    "minimax_small_tnd": (_custom("minimax_small", 1, 2, 2, 128, 512, (6, 24, 42), False, 0.8),
                          {"layout": "TND"}),
    # sparsity 0.5, D=64, GQA 2/1, batch 2
    "b2_gqa_d64": (_custom("b2_gqa_d64", 2, 2, 1, 64, 77, (5, 16, 40), True, 0.5), {}),
    # dense fallback: 31 sparse blocks (below 32) and exactly 32
    "fallback_31": (_custom("fallback_31", 1, 2, 2, 64, 128, (3, 8, 248), True, 0.8), {}),
    "sparse_32": (_custom("sparse_32", 1, 2, 2, 64, 128, (3, 8, 256), True, 0.8), {}),
    # sparsity 0 disables sparsity
    "sparsity0": (_custom("sparsity0", 1, 2, 2, 128, 128, (9, 16, 32), True, 0.0), {}),
    # fp8 precision: D=64, and ragged GQA D=128 in TND with batch 2
    "tiny_fp8": (WORKLOADS["tiny"].with_(precision="fp8"), {}),
    "ragged_gqa_fp8": (_custom("ragged_gqa", 1, 4, 2, 128, 200, (10, 17, 34), True, 0.8,
                               precision="fp8"), {}),
    "minimax_small_fp8_tnd_b2": (_custom("minimax_small", 2, 2, 2, 128, 512, (6, 24, 42), False,
                                         0.8, precision="fp8"), {"layout": "TND"}),
    # mxfp4 precision: D=64; ragged GQA D=128; a 32-row last block in TND with batch 2
    "tiny_mxfp4": (WORKLOADS["tiny"].with_(precision="mxfp4"), {}),
    "ragged_gqa_mxfp4": (_custom("ragged_gqa", 1, 4, 2, 128, 200, (10, 17, 34), True, 0.8,
                                 precision="mxfp4"), {}),
    "minimax_small_mxfp4_tnd_b2": (_custom("minimax_small", 2, 2, 2, 128, 512, (6, 24, 42), False,
                                           0.8, precision="mxfp4"), {"layout": "TND"}),
    # no geometry at all: dense over a sequence that is not a multiple of 128
    "no_grid": (_custom("no_grid", 1, 2, 2, 128, 1000, (0, 0, 0), False, 0.8), {"grid": (0, 0, 0)}),
}


def _inputs(w, layout):
    return case_inputs(w, layout)


def _desc(w, extra):
    return case_desc(w, extra)


def _full_check(name):
    return full_check(*SMALL[name], name=name)


@pytest.mark.parametrize("name", [mx_param(n) for n in sorted(SMALL)])
def test_small_case(name):
    _full_check(name)


def test_dense_cases_equal_dense_attention():
    """Fallback and sparsity 0 lists are all dense, so the output is plain attention."""
    import torch
    for name in ("fallback_31", "sparsity0", "no_grid"):
        w, extra = SMALL[name]
        desc = _desc(w, extra)
        q, k, v = _inputs(w, "BNSD")
        res = run_gpu(desc, q, k, v)
        assert res["bufs"].info.dense_fallback == 1
        ref = torch.nn.functional.scaled_dot_product_attention(
            *(torch.from_numpy(f32(x).astype(np.float64)) for x in (q, k, v))).numpy()
        assert_close(f32(to_host_u16(res["out"])), ref, BF16_TOL, f"{name} vs torch SDPA")


@pytest.mark.parametrize("precision", [mx_param(x) for x in ("bf16", "mix", "fp8", "mxfp4")])
def test_empty_lists_give_zeros(precision):
    """Sparsity 1, no prefix, no first frame, aligned grid: every list is empty."""
    w = _custom("empty", 1, 2, 2, 128, 0, (4, 16, 16), False, 1.0, precision=precision)
    import block_sparse_video_rf_amd as rf
    desc = rf.Desc.from_workload(w, min_sparse_blocks=1)
    q, k, v = make_qkv(w)
    res = run_gpu(desc, q, k, v)
    assert int(res["bufs"].select_num.max()) == 0
    assert np.all(to_host_u16(res["out"]) == 0)


@pytest.mark.parametrize("precision", [mx_param(x) for x in ("bf16", "mix", "fp8", "mxfp4")])
def test_handmade_lists_skip_invalid_entries(precision):
    """rf_sparse_attn accepts any list: -1 and out-of-range ids are skipped, counts clamped."""
    import torch
    import block_sparse_video_rf_amd as rf
    w = SMALL["minimax_small"][0].with_(precision=precision)
    desc = rf.Desc.from_workload(w)
    q, k, v = make_qkv(w)
    res = run_gpu(desc, q, k, v)
    b = res["bufs"]
    nB = b.info.n_blocks
    rng = np.random.default_rng(3)
    idx = np.full((nB, w.heads_q, nB), -1, dtype=np.int32)
    num = np.zeros((nB, w.heads_q), dtype=np.int32)
    valid_idx = np.full_like(idx, -1)
    valid_num = np.zeros_like(num)
    for qb in range(nB):
        for n in range(w.heads_q):
            m = int(rng.integers(0, 12))
            ids = rng.choice(nB, size=m, replace=False)
            lst = list(ids) + [-1, nB + 5, 10 ** 6]
            rng.shuffle(lst)
            idx[qb, n, :len(lst)] = lst
            # Some counts run past the list width: the kernel clamps them to
            # max_kv, so every entry of the row (the -1 fill included) counts.
            num[qb, n] = len(lst) + (nB + 5 if qb % 7 == 0 else 0)
            good = [x for x in lst if 0 <= x < nB]
            valid_idx[qb, n, :len(good)] = good
            valid_num[qb, n] = len(good)
    assert (num > nB).any()
    out_p = torch.empty_like(b.out_p)
    rf.rf_sparse_attn(desc, b.qp, b.kp, b.vpt, b.q8, b.k8, b.q_scale, b.k_scale, b.v_scale,
                      torch.from_numpy(idx).cuda(), torch.from_numpy(num).cuda(), nB, out_p)
    torch.cuda.synchronize()
    g = geometry_of(desc)
    # The oracle on the valid entries only, with the precision's own quantisation.
    ores = oracle.run(f32(q), f32(k), f32(v), g, precision=precision,
                      select=(valid_idx, valid_num))
    ref = ores["out_p"]
    if precision in ("fp8", "mxfp4"):
        assert_within(f32(to_host_u16(out_p)), ref,
                      fp8_bound_permuted(ores, (valid_idx, valid_num)),
                      f"handmade lists ({precision})")
    else:
        assert_close(f32(to_host_u16(out_p)), ref, BF16_TOL, f"handmade lists ({precision})")


def test_recomputed_pools_and_determinism():
    """rf_pool_select without pooled inputs recomputes them; two runs are bit-identical."""
    import torch
    import block_sparse_video_rf_amd as rf
    w, _ = SMALL["ragged_gqa"]
    desc = rf.Desc.from_workload(w)
    q, k, v = make_qkv(w)
    r1 = run_gpu(desc, q, k, v)
    r2 = run_gpu(desc, q, k, v)
    assert torch.equal(r1["out"], r2["out"])
    assert torch.equal(r1["bufs"].select_idx, r2["bufs"].select_idx)
    b = r1["bufs"]
    idx2 = torch.empty_like(b.select_idx)
    num2 = torch.empty_like(b.select_num)
    rf.rf_pool_select(desc, b.qp, b.kp, None, None, idx2, num2, b.info.n_blocks, b.workspace)
    torch.cuda.synchronize()
    assert torch.equal(idx2, b.select_idx) and torch.equal(num2, b.select_num)


_SEL_COUNTS = [32, 64, 65, 511, 512, 513, 1024, 1025, 2048, 2049]


@pytest.mark.parametrize("grid", [(5, 16, 1200), (3, 16, 8400), (3, 8, 65536)]
                         + [(3, 8, 8 * n) for n in _SEL_COUNTS],
                         ids=["nS600", "nS2100", "nS8192"] + [f"nS{n}" for n in _SEL_COUNTS])
def test_selection_paths_by_sparse_count(grid):
    """Selection alone at 600 sparse blocks (16 keys per lane), at 2100 (above
    the register path: one workgroup per row) and at 8192 (the largest accepted,
    the workgroup path's LDS full), and on both sides of every dispatch
    boundary (8, 16 and 32 keys per lane up to 512, 1024 and 2048 blocks; one
    key per lane at 64), against the oracle's rule."""
    import torch
    import block_sparse_video_rf_amd as rf
    w = _custom("sel", 1, 1, 1, 64, 128, grid, True, 0.8)
    desc = rf.Desc.from_workload(w)
    log(f"[selection nS] grid={grid} S={w.seq_len}")
    q, k, v = make_qkv(w)
    b = rf.Buffers(desc)
    rf.rf_permute(desc, *(torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(
        torch.bfloat16).cuda() for x in (q, k, v)), b.qp, b.kp, b.vpt, b.q_pool, b.k_pool)
    rf.rf_pool_select(desc, b.qp, b.kp, b.q_pool, b.k_pool, b.select_idx, b.select_num,
                      b.info.n_blocks, b.workspace)
    torch.cuda.synchronize()
    g = geometry_of(desc)
    p = plan(g)
    assert p.n_sparse == b.info.n_sparse == grid[1] // 8 * grid[2] // 8 * ((grid[0] - 1) // 2)
    pi = permutation(g)
    qpool = oracle.pool_blocks(f32(oracle.permute_rows(q, pi)), p)
    kpool = oracle.pool_blocks(f32(oracle.permute_rows(k, pi)), p)
    scores = oracle.block_scores(qpool, kpool, 1.0 / np.sqrt(w.head_dim))
    swaps = check_selection(p, 1, 1, b.select_idx.cpu().numpy(), b.select_num.cpu().numpy(),
                            scores)
    log(f"  selection exact ({swaps} near-tie rows)")


@pytest.mark.parametrize("precision", [mx_param(x) for x in ("bf16", "mix", "fp8", "mxfp4")])
def test_reference_raised_mid_row(precision):
    """Keys in the second half of the sequence scaled by 100: their logits exceed
    the reference the first blocks set by far more than 2^64 allows, so the
    softmax raises it (and rescales) in the middle of every row."""
    import block_sparse_video_rf_amd as rf
    from synth import bf16_from_f32
    w = _custom("grow", 1, 2, 2, 64, 128, (9, 16, 32), True, 0.0, precision=precision)
    desc = rf.Desc.from_workload(w)
    q, k, v = make_qkv(w)
    kf = f32(k)
    half = w.seq_len // 2
    kf[:, :, half:, :] *= 100.0
    k = bf16_from_f32(kf)
    res = run_gpu(desc, q, k, v)
    assert res["bufs"].info.dense_fallback == 1   # every block listed, in order
    g = geometry_of(desc)
    ores = oracle.run(f32(q), f32(k), f32(v), g, precision=precision)
    ref = ores["out"]
    # Logits this large make every row peaked, so little averaging hides the bf16
    # rounding of P (2^-9 relative) and of the output: together at most
    # 2^-9 * (max|v - O| + |O|), about 2.4e-2 for |v| <= 4. A wrong rescale
    # would show in the mean, which keeps its bound. fp8: the derived
    # per-element bound (peaked rows carry large P shares, so a flipped code or
    # the one-pass subnormal rounding weighs more there; the bound follows).
    if precision in ("fp8", "mxfp4"):
        kb = in_output_layout(fp8_bound_permuted(ores, (ores["select_idx"], ores["select_num"])),
                              ores)
        assert_within(f32(to_host_u16(res["out"])), ref, kb, f"raised mid-row ({precision})")
        return
    assert_close(f32(to_host_u16(res["out"])), ref, (4e-2, BF16_TOL[1]),
                 f"raised mid-row ({precision})")
