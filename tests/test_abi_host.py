"""Host-side tests of the C ABI (no GPU needed).

* the library loads and exports every function include/rf.h declares;
* rf_plan (host-only) agrees with the oracle's geometry on random
  geometries and on the five workloads;
* every validation error is reported by rf_plan and by each entry point
  before anything is enqueued (these calls never reach a HIP launch).
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import block_sparse_video_rf_amd as rf
from block_sparse_video_rf_amd.rf import RfDesc, RfError, load_library
from oracle.geometry import Geometry, plan
from synth import WORKLOADS

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "rf.h")


def test_exports_every_declared_symbol():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:rf_status|const char\*)\s+(rf_\w+)\(", text, re.M))
    assert declared == set(rf.EXPORTS)
    lib = load_library()
    for name in declared:
        assert hasattr(lib, name), name
    assert "gfx950" in rf.rf_version()


def _check_plan(desc, g):
    info = rf.rf_plan(desc)
    p = plan(g)
    assert info.dense_fallback == int(p.fallback)
    assert (info.n_head, info.n_sparse, info.n_tail) == (p.n_head, p.n_sparse, p.n_tail)
    assert info.n_blocks == p.n_blocks == info.max_kv_blocks
    assert info.topk == p.topk
    assert info.head_rows == p.head_rows
    assert info.sparse_rows == p.sparse_rows
    assert info.promoted_rows == p.promoted_rows
    assert info.select_rows == desc.batch * p.n_blocks
    assert info.vpt_elems == desc.batch * desc.heads_kv * p.n_blocks * desc.head_dim * 128


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_plan_matches_oracle_workloads(name):
    w = WORKLOADS[name]
    _check_plan(rf.Desc.from_workload(w), Geometry(w.prefix_len, w.grid, w.first_frame, w.sparsity))


def test_plan_matches_oracle_random_geometries():
    rng = np.random.default_rng(2024)
    for _ in range(400):
        T = int(rng.integers(1, 12))
        H = int(rng.integers(1, 40))
        W = int(rng.integers(1, 40))
        P = int(rng.integers(0, 400))
        f0 = bool(rng.integers(0, 2))
        s = float(rng.choice([0.0, 0.3, 0.5, 0.8, 0.9, 1.0]))
        mb = int(rng.choice([1, 4, 32]))
        desc = rf.Desc(batch=1, heads_q=2, heads_kv=1, head_dim=64, seq_len=P + T * H * W,
                       prefix_len=P, first_frame_rows=H * W if f0 else 0, grid=(T, H, W),
                       sparsity=s, min_sparse_blocks=mb)
        _check_plan(desc, Geometry(P, (T, H, W), f0, s, min_sparse_blocks=mb))


def test_plan_without_geometry_is_dense():
    info = rf.rf_plan(rf.Desc(batch=2, heads_q=4, heads_kv=4, head_dim=128, seq_len=1000))
    assert info.dense_fallback == 1 and info.n_blocks == 8 and info.n_sparse == 0
    assert info.ws_select_bytes == 0


def _good():
    w = WORKLOADS["tiny"]
    return rf.Desc.from_workload(w)


BAD = [
    ("layout", dict(layout=7), 2),
    ("dtype", dict(dtype=1), 3),
    ("batch", dict(batch=0), 4),
    ("heads", dict(heads_q=0), 4),
    ("seq", dict(seq_len=0), 4),
    ("seq_bytes", dict(seq_len=1 << 24), 4),  # 2^24 rows x 64 x 2 B = 2 GiB per head
    ("scale", dict(scale=-1.0), 4),
    ("scale_nan", dict(scale=float("nan")), 4),
    ("block_zero", dict(block_shape=(0, 128)), 5),
    ("block_64", dict(block_shape=(64, 64)), 10),
    ("head_dim", dict(head_dim=96), 10),
    ("gqa", dict(heads_q=3, heads_kv=2), 6),
    ("sparsity_neg", dict(sparsity=-0.1), 7),
    ("sparsity_big", dict(sparsity=1.5), 7),
    ("sparsity_nan", dict(sparsity=float("nan")), 7),
    ("sparsity_inf", dict(sparsity=float("inf")), 7),
    ("geometry_len", dict(seq_len=4737), 8),
    ("geometry_ff", dict(first_frame_rows=100), 8),
    ("geometry_grid", dict(grid=(9, 0, 32)), 8),
    ("precision_bad", dict(precision=9), 11),
    # 8193 sparse blocks (one 8-row strip of 8193 tiles): one more than the
    # selection kernel holds
    ("sparse_limit", dict(grid=(3, 8, 8 * 8193), first_frame_rows=8 * 8 * 8193,
                          seq_len=128 + 3 * 8 * 8 * 8193), 10),
]


def test_sparse_block_limit_accepted():
    """Exactly 8192 sparse blocks is the largest accepted geometry."""
    d = _good()
    d.grid = (3, 8, 8 * 8192)
    d.first_frame_rows = 8 * 8 * 8192
    d.seq_len = 128 + 3 * 8 * 8 * 8192
    info = rf.rf_plan(d)
    assert info.n_sparse == 8192 and info.dense_fallback == 0


@pytest.mark.parametrize("name,change,status", BAD, ids=[b[0] for b in BAD])
def test_invalid_descriptors(name, change, status):
    d = _good()
    for k_, v_ in change.items():
        setattr(d, k_, v_)
    with pytest.raises(RfError) as e:
        rf.rf_plan(d)
    assert e.value.status == status
    # Every entry point validates the descriptor first and enqueues nothing.
    lib = load_library()
    c = d.c()
    fake = ctypes.c_void_p(0x1000)
    assert lib.rf_permute(ctypes.byref(c), fake, fake, fake, fake, fake, fake, None, None, None,
                          None, None, None, None, None) == status
    assert lib.rf_pool_select(ctypes.byref(c), fake, fake, None, None, fake, fake, 1000, fake,
                              1 << 30, None) == status
    assert lib.rf_sparse_attn(ctypes.byref(c), fake, fake, fake, None, None, None, None, None,
                              fake, fake, 1000, fake, None) == status
    assert lib.rf_dense_attn(ctypes.byref(c), fake, fake, fake, None, None, None, None, None,
                             fake, None) == status
    assert lib.rf_unpermute(ctypes.byref(c), fake, fake, None) == status


def test_mxfp4_sizes_planned_and_buffers_checked():
    """rf_plan reports the mxfp4 buffer sizes; the device entry points check the
    buffers mxfp4 needs before any launch (RF_ERR_PRECISION without them)."""
    d = _good()
    d.precision = "mxfp4"
    info = rf.rf_plan(d)
    B, N1, N2, S, D = d.batch, d.heads_q, d.heads_kv, d.seq_len, d.head_dim
    # Natural sizes: no buffer is read past its real rows.
    assert info.q8_bytes == B * N1 * S * D // 2 and info.k8_bytes == B * N2 * S * D // 2
    assert info.q_scale_bytes == B * N1 * S * D // 32
    assert info.k_scale_bytes == B * N2 * S * D // 32
    assert info.kp_bytes == 2 * B * N2 * S * D
    assert info.vpt_bytes == B * N2 * info.n_blocks * D * 64
    assert info.v_scale_bytes == B * N2 * info.n_blocks * 4 * D
    lib = load_library()
    c = d.c()
    fake = ctypes.c_void_p(1 << 40)
    # Q without its E8M0 scales; V without its scales; attention without V scales.
    assert lib.rf_permute(ctypes.byref(c), fake, None, None, None, None, None, None, None,
                          ctypes.c_void_p(2 << 40), None, None, None, None, None) == 11
    assert lib.rf_permute(ctypes.byref(c), None, None, fake, None, None,
                          ctypes.c_void_p(2 << 40), None, None, None, None, None, None, None,
                          None) == 11
    assert lib.rf_sparse_attn(ctypes.byref(c), None, None, fake, fake, fake, fake, fake, None,
                              fake, fake, info.n_blocks, ctypes.c_void_p(5 << 40), None) == 11
    assert lib.rf_dense_attn(ctypes.byref(c), None, None, fake, fake, fake, fake, fake, None,
                             ctypes.c_void_p(5 << 40), None) == 11
    # Per-precision sizes of the other modes.
    for prec, q8, vpt in (("bf16", 0, 2), ("mix", 1, 2), ("fp8", 1, 1)):
        d.precision = prec
        i = rf.rf_plan(d)
        assert i.q8_bytes == q8 * i.qp_elems and i.vpt_bytes == vpt * i.vpt_elems
        assert i.k8_bytes == q8 * i.kp_elems and i.kp_bytes == 2 * i.kp_elems


def test_status_strings():
    for s in range(15):
        assert rf.rf_status_str(s) and rf.rf_status_str(s) != "unknown status"
    assert rf.rf_status_str(99) == "unknown status"


def test_argument_errors_before_launch():
    lib = load_library()
    d = _good()
    c = d.c()
    info = rf.rf_plan(d)
    big = 1 << 40
    P = ctypes.c_void_p
    a, b2, c3, d4, e5 = (P(big * i) for i in range(1, 6))
    # NULL descriptor / info.
    assert lib.rf_plan(None, None) == 1
    assert lib.rf_plan(ctypes.byref(c), None) == 1
    # rf_permute: V without its block-transposed output.
    assert lib.rf_permute(ctypes.byref(c), None, None, a, None, None, None, None, None, None,
                          None, None, None, None, None) == 1
    # rf_permute: output overlapping its input.
    assert lib.rf_permute(ctypes.byref(c), a, None, None, a, None, None, None, None, None, None,
                          None, None, None, None) == 13
    # rf_permute in fp8: V without its power-of-two scales; Q without its codes.
    d8 = _good()
    d8.precision = "fp8"
    c8 = d8.c()
    assert lib.rf_permute(ctypes.byref(c8), None, None, a, None, None, b2, None, None, None,
                          None, None, None, None, None) == 11
    assert lib.rf_permute(ctypes.byref(c8), a, None, None, b2, None, None, None, None, None,
                          None, None, None, None, None) == 11
    # rf_pool_select: workspace too small, NULL workspace, narrow selectIdx.
    assert lib.rf_pool_select(ctypes.byref(c), a, b2, None, None, c3, d4, info.n_blocks, e5,
                              info.ws_select_bytes - 1, None) == 9
    assert lib.rf_pool_select(ctypes.byref(c), a, b2, None, None, c3, d4, info.n_blocks, None,
                              info.ws_select_bytes, None) == 1
    assert lib.rf_pool_select(ctypes.byref(c), a, b2, None, None, c3, d4, info.n_blocks - 1, e5,
                              info.ws_select_bytes, None) == 4
    # rf_sparse_attn: mix precision without its fp8 buffers; output aliasing Q.
    dm = _good()
    dm.precision = "mix"
    cm = dm.c()
    assert lib.rf_sparse_attn(ctypes.byref(cm), a, b2, c3, None, None, None, None, None, d4, e5,
                              info.n_blocks, P(big * 7), None) == 11
    assert lib.rf_sparse_attn(ctypes.byref(c), a, b2, c3, None, None, None, None, None, d4, e5,
                              info.n_blocks, a, None) == 13
    assert lib.rf_sparse_attn(ctypes.byref(c), a, b2, c3, None, None, None, None, None, d4, e5,
                              0, P(big * 7), None) == 4
    # fp8: every mix buffer but the V scales is not enough; with them the output
    # may not overlap the scales.
    f1, f2, f3, f4 = (P(big * i) for i in range(8, 12))
    assert lib.rf_sparse_attn(ctypes.byref(c8), None, None, c3, f1, f2, f3, f4, None, d4, e5,
                              info.n_blocks, P(big * 7), None) == 11
    assert lib.rf_dense_attn(ctypes.byref(c8), None, None, c3, f1, f2, f3, f4, None,
                             P(big * 7), None) == 11
    assert lib.rf_dense_attn(ctypes.byref(c8), None, None, c3, f1, f2, f3, f4, P(big * 12),
                             P(big * 12), None) == 13
    # rf_unpermute: NULL output, aliasing output.
    assert lib.rf_unpermute(ctypes.byref(c), a, None, None) == 1
    assert lib.rf_unpermute(ctypes.byref(c), a, a, None) == 13
    # Nothing to do is not an error: all inputs NULL.
    assert lib.rf_permute(ctypes.byref(c), None, None, None, None, None, None, None, None, None,
                          None, None, None, None, None) == 0


def test_pool_select_overlap_checks():
    """rf_pool_select and its no-allocation form refuse lists or a workspace that
    overlap what the call reads (the pooled blocks, or the rows they are pooled
    from), before any launch."""
    lib = load_library()
    d = _good()
    c = d.c()
    info = rf.rf_plan(d)
    P = ctypes.c_void_p
    big = 1 << 40
    qp, kp, qpool, kpool, idx, num, ws = (P(big * i) for i in range(1, 8))
    nb = info.n_blocks
    wsb = info.ws_select_bytes
    # Workspace on top of the pooled Q blocks, of K, or of the lists.
    assert lib.rf_pool_select(ctypes.byref(c), None, None, qpool, kpool, idx, num, nb, qpool,
                              wsb, None) == 13
    assert lib.rf_pool_select(ctypes.byref(c), None, kp, qpool, None, idx, num, nb, kp, wsb,
                              None) == 13
    assert lib.rf_pool_select(ctypes.byref(c), None, None, qpool, kpool, idx, num, nb, idx, wsb,
                              None) == 13
    # selectIdx over the pooled K blocks; selectNum inside selectIdx.
    assert lib.rf_pool_select(ctypes.byref(c), None, None, qpool, kpool, kpool, num, nb, ws,
                              wsb, None) == 13
    assert lib.rf_pool_select(ctypes.byref(c), None, None, qpool, kpool, idx, P(5 * big + 64), nb,
                              ws, wsb, None) == 13
    assert lib.rf_pool_select_noalloc(ctypes.byref(c), qp, kp, None, None, qp, num, nb,
                                      None) == 13
    # qp is not read when the pooled Q blocks are given: no overlap to report.
    assert lib.rf_pool_select(ctypes.byref(c), idx, None, qpool, kpool, idx, num, nb, ws, wsb,
                              None) != 13


def test_pool_select_noalloc_refuses_oversized_scratch():
    """A call whose block scores do not fit the fixed device array returns
    RF_ERR_SCRATCH before touching any device (16 heads x 1440^2 scores > 72 MiB);
    with the pooled blocks recomputed the pieces add up (the layout of rf_plan's
    workspace)."""
    lib = load_library()
    d = rf.Desc(batch=1, heads_q=16, heads_kv=2, head_dim=128, seq_len=512 + 31 * 64 * 96,
                prefix_len=512, first_frame_rows=64 * 96, grid=(31, 64, 96), sparsity=0.9)
    info = rf.rf_plan(d)
    assert info.n_sparse == 1440
    scores = 16 * 1440 * 1440 * 4
    assert scores > rf.NOALLOC_SCRATCH_BYTES
    P = ctypes.c_void_p
    big = 1 << 40
    c = d.c()
    assert lib.rf_pool_select_noalloc(ctypes.byref(c), None, None, P(big), P(2 * big), P(3 * big),
                                      P(4 * big), info.n_blocks, None) == 14
    assert "scratch" in rf.rf_status_str(14)
    # The long GQA workload fits, pools recomputed included.
    w = WORKLOADS["gqa_long"]
    i2 = rf.rf_plan(rf.Desc.from_workload(w))
    assert i2.ws_select_bytes <= rf.NOALLOC_SCRATCH_BYTES
