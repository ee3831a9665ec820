"""rf_pool_select_noalloc, the selection entry point for callers that cannot
allocate, against rf_pool_select on the same inputs.

Both run the same pool, score and select kernels; the no-allocation form only
takes its workspace from the library's fixed device array. Two calls in a row,
the second on a smaller input (so the array still holds the first call's
scores and pools): the lists must be identical, bit for bit, each time. The
first call recomputes the pooled blocks (the largest use of the array: the
long GQA workload's 8 x 1440 x 1440 scores plus both pools); the second uses
pooled blocks from rf_permute. Free device memory is unchanged across a
no-allocation call.
"""
import numpy as np
import pytest

from synth import WORKLOADS, make_qkv

from gpu_harness import log, to_dev

pytestmark = pytest.mark.gpu


def _inputs(desc, w):
    import block_sparse_video_rf_amd as rf
    q, k, _ = make_qkv(w)
    bufs = rf.Buffers(desc)
    rf.rf_permute(desc, to_dev(q), to_dev(k), None, bufs.qp, bufs.kp, None, bufs.q_pool,
                  bufs.k_pool)
    return bufs


def _compare(name, recompute_pools):
    import torch
    import block_sparse_video_rf_amd as rf
    w = WORKLOADS[name]
    desc = rf.Desc.from_workload(w)
    bufs = _inputs(desc, w)
    info = bufs.info
    nB = info.n_blocks
    q_pool = None if recompute_pools else bufs.q_pool
    k_pool = None if recompute_pools else bufs.k_pool
    rf.rf_pool_select(desc, bufs.qp, bufs.kp, q_pool, k_pool, bufs.select_idx, bufs.select_num,
                      nB, bufs.workspace)
    idx = torch.full_like(bufs.select_idx, -7)
    num = torch.full_like(bufs.select_num, -7)
    torch.cuda.synchronize()
    free_before = torch.cuda.mem_get_info()[0]
    rf.rf_pool_select_noalloc(desc, bufs.qp, bufs.kp, q_pool, k_pool, idx, num, nB)
    torch.cuda.synchronize()
    free_after = torch.cuda.mem_get_info()[0]
    assert free_after == free_before, (free_before, free_after)
    ref_idx, ref_num = bufs.select_idx.cpu().numpy(), bufs.select_num.cpu().numpy()
    got_idx, got_num = idx.cpu().numpy(), num.cpu().numpy()
    assert np.array_equal(got_num, ref_num)
    assert np.array_equal(got_idx, ref_idx)
    # The lists are real selections: sparse rows keep head + topk + tail blocks.
    sparse_rows = slice(info.n_head, info.n_head + info.n_sparse)
    assert np.all(ref_num[sparse_rows] == info.n_head + info.topk + info.n_tail)
    log(f"  {name}: {ref_idx.shape[0]} x {ref_idx.shape[1]} lists identical "
        f"(pools {'recomputed' if recompute_pools else 'given'}, "
        f"workspace {info.ws_select_bytes / 2**20:.1f} MiB of "
        f"{rf.NOALLOC_SCRATCH_BYTES / 2**20:.0f} MiB)")


def test_noalloc_matches_pool_select_twice():
    log("[no-alloc] gqa_long with pools recomputed, then tiny with pools given")
    _compare("gqa_long", recompute_pools=True)
    _compare("tiny", recompute_pools=False)
