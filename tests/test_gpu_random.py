"""GPU parity on a seeded sweep of random small geometries: every step of the
path against the oracle, with the contract of the small cases (bit-exact
arrangement, codes and selection; attention within its precision's bounds).

Each case draws: prefix length (0, 1, 77, 128, 200, 300), latent grid
(T in [2, 6], H and W in [8, 24]: unaligned widths, odd frame counts),
first-frame sink on or off, sparsity (0.3, 0.5, 0.8, 0.95), head dim (64,
128), GQA ratio (1, 2), one or two kv heads, batch (1, 2), layout (BNSD, TND),
precision (bf16, mix, fp8), and smooth or plain inputs. The sparse path is
taken from one sparse block up (min_sparse_blocks = 1)."""
import numpy as np
import pytest

from synth import Workload

from gpu_harness import full_check, log

pytestmark = pytest.mark.gpu


def _case(seed):
    rng = np.random.default_rng(7000 + seed)
    D = int(rng.choice([64, 128]))
    N2 = int(rng.integers(1, 3))
    G = int(rng.choice([1, 2]))
    B = int(rng.choice([1, 2])) if N2 * G <= 2 else 1
    grid = (int(rng.integers(2, 7)), int(rng.integers(8, 25)), int(rng.integers(8, 25)))
    P = int(rng.choice([0, 1, 77, 128, 200, 300]))
    f0 = bool(rng.integers(0, 2))
    s = float(rng.choice([0.3, 0.5, 0.8, 0.95]))
    prec = str(rng.choice(["bf16", "mix", "fp8"]))
    layout = str(rng.choice(["BNSD", "TND"]))
    smooth = bool(rng.integers(0, 2))
    w = Workload(f"random{seed}", B, N2 * G, N2, D, P, grid, f0, s, prec, smooth, 9000 + seed)
    return w, {"layout": layout, "min_sparse_blocks": 1}


# Seeds 0-9, and six mix cases of a wider one-off sweep (200 seeds) where the
# oracle's own E4M3 Q/K result deviates 6.2e-2 to 9.9e-2 (max-abs) from the
# unquantised one: the end-to-end bar then follows that deviation.
@pytest.mark.parametrize("seed", list(range(10)) + [15, 74, 75, 88, 126, 202])
def test_random_geometry(seed):
    w, extra = _case(seed)
    log(f"[random {seed}] {w}")
    full_check(w, extra)


def _prepared(seed):
    """A case's inputs run through the path once (fills the permuted buffers)."""
    import block_sparse_video_rf_amd as rf
    from gpu_harness import case_desc, case_inputs, to_dev
    w, extra = _case(seed)
    desc = case_desc(w, extra)
    q, k, v = case_inputs(w, extra["layout"])
    out, b = rf.attention(to_dev(q), to_dev(k), to_dev(v), desc)
    return w, desc, (q, k, v), b


@pytest.mark.parametrize("seed", range(10))
def test_random_dense_entry_equals_every_block_listed(seed):
    import torch
    import block_sparse_video_rf_amd as rf
    w, desc, _, b = _prepared(seed)
    nB = b.info.n_blocks
    rows = w.batch * nB
    idx = torch.arange(nB, dtype=torch.int32, device="cuda").repeat(rows, w.heads_q, 1)
    num = torch.full((rows, w.heads_q), nB, dtype=torch.int32, device="cuda")
    o_sparse = torch.empty_like(b.out_p)
    o_dense = torch.empty_like(b.out_p)
    rf.rf_sparse_attn(desc, b.qp, b.kp, b.vpt, b.q8, b.k8, b.q_scale, b.k_scale, b.v_scale, idx,
                      num, nB, o_sparse)
    rf.rf_dense_attn(desc, b.qp, b.kp, b.vpt, b.q8, b.k8, b.q_scale, b.k_scale, b.v_scale, o_dense)
    torch.cuda.synchronize()
    assert torch.equal(o_sparse.view(torch.int16), o_dense.view(torch.int16))


@pytest.mark.parametrize("seed", range(10))
def test_random_lists_with_invalid_entries(seed):
    """Unsorted lists of random blocks mixed with -1 and out-of-range ids, and
    counts past the list width (clamped), against the oracle on the valid ids."""
    import torch
    import block_sparse_video_rf_amd as rf
    import oracle
    from gpu_harness import (BF16_TOL, assert_close, assert_within, f32, fp8_bound_permuted,
                             geometry_of, to_host_u16)
    w, desc, (q, k, v), b = _prepared(seed)
    nB = b.info.n_blocks
    rows = w.batch * nB
    rng = np.random.default_rng(100 + seed)
    idx = np.full((rows, w.heads_q, nB), -1, dtype=np.int32)
    num = np.zeros((rows, w.heads_q), dtype=np.int32)
    valid_idx = np.full_like(idx, -1)
    valid_num = np.zeros_like(num)
    for r in range(rows):
        for n in range(w.heads_q):
            m = int(rng.integers(0, min(nB, 9) + 1))
            lst = list(rng.choice(nB, size=m, replace=False))
            junk = [-1, nB, nB + 7, -5][:int(rng.integers(0, 3))]
            lst = lst + junk
            rng.shuffle(lst)
            lst = lst[:nB]
            idx[r, n, :len(lst)] = lst
            num[r, n] = min(len(lst) + int(rng.integers(0, 3)), nB)   # a count past the entries
            good = [x for x in lst[:num[r, n]] if 0 <= x < nB]
            valid_idx[r, n, :len(good)] = good
            valid_num[r, n] = len(good)
    out_p = torch.empty_like(b.out_p)
    rf.rf_sparse_attn(desc, b.qp, b.kp, b.vpt, b.q8, b.k8, b.q_scale, b.k_scale, b.v_scale,
                      torch.from_numpy(idx).cuda(), torch.from_numpy(num).cuda(), nB, out_p)
    torch.cuda.synchronize()
    from synth import from_tnd
    qb, kb, vb = (from_tnd(x, w.batch) if desc.layout == "TND" else x for x in (q, k, v))
    ores = oracle.run(f32(qb), f32(kb), f32(vb), geometry_of(desc), precision=w.precision,
                      select=(valid_idx, valid_num), batch=w.batch)
    ref = ores["out_p"]
    if w.precision == "fp8":
        assert_within(f32(to_host_u16(out_p)), ref,
                      fp8_bound_permuted(ores, (valid_idx, valid_num)), "random lists (fp8)")
    else:
        assert_close(f32(to_host_u16(out_p)), ref, BF16_TOL, f"random lists ({w.precision})")
