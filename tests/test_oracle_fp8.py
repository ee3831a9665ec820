"""Pins of the oracle's OCP E4M3 codec and the mix-precision block quantiser.

The codec is checked against PyTorch's CPU ``float8_e4m3fn`` conversion (an
independent implementation of the same OCP format) on all 256 codes, on
random values and on every rounding midpoint; saturation beyond 448 (where
PyTorch produces NaN instead) is checked against its closed form.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.fp8 import E4M3_MAX, e4m3_decode, e4m3_encode, quantize_blocks
from oracle.geometry import Geometry, plan


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_decode_all_codes():
    mine = e4m3_decode(np.arange(256, dtype=np.uint8))
    ref = _torch_decode_all()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.nanmax(mine) == E4M3_MAX
    assert mine[1] == 2.0 ** -9 and mine[8] == 2.0 ** -6


def test_encode_inverts_decode():
    vals = e4m3_decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        if np.isnan(vals[c]):
            continue
        assert e4m3_encode(np.array([vals[c]]))[0] == c


def test_encode_matches_torch_random_and_midpoints():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1, 30, 200)])
    x = x[np.abs(x) <= E4M3_MAX].astype(np.float32)
    assert np.array_equal(e4m3_encode(x), _torch_encode(x))
    vals = np.unique(np.abs(_torch_decode_all()[~np.isnan(_torch_decode_all())]))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    mids = np.concatenate([mids, -mids])
    assert np.array_equal(e4m3_encode(mids), _torch_encode(mids))


def test_saturation_closed_form():
    big = np.array([448.0, 449.0, 463.99, 464.0, 500.0, 1e6, 3e38], dtype=np.float64)
    assert np.all(e4m3_decode(e4m3_encode(big)) == 448.0)
    assert np.all(e4m3_decode(e4m3_encode(-big)) == -448.0)


def test_quantize_blocks_properties():
    g = Geometry(512, (6, 24, 42), False, 0.8, min_sparse_blocks=1)  # short last block
    p = plan(g)
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((1, 2, g.seq_len, 16)) * 3).astype(np.float32)
    r0z, nz = p.blocks[2]
    x[0, 1, r0z:r0z + nz] = 0.0                                   # an all-zero block
    codes, sigma = quantize_blocks(x, p)
    for j, (r0, n) in enumerate(p.blocks):
        for h in range(2):
            blk = x[0, h, r0:r0 + n]
            amax = np.float32(np.abs(blk).max())
            if amax == 0:
                assert sigma[0, h, j] == 1 and np.all(codes[0, h, r0:r0 + n] == 0)
                continue
            assert sigma[0, h, j] == np.float32(amax / np.float32(448))
            deq = e4m3_decode(codes[0, h, r0:r0 + n]) * sigma[0, h, j]
            # The block maximum lands on the top code; the rest within half a quantum
            # (relative 2**-4 for normals, absolute 2**-10 * sigma for subnormals).
            assert np.abs(e4m3_decode(codes[0, h, r0:r0 + n])).max() == 448.0
            err = np.abs(deq - blk)
            assert np.all(err <= np.maximum(np.abs(blk) * 2.0 ** -4, 2.0 ** -10 * sigma[0, h, j]) * 1.0001)


def test_mix_pipeline_equals_dequantised_bf16_pipeline():
    g = Geometry(128, (9, 16, 32), True, 0.8)
    S = g.seq_len
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((1, 2, S, 16)).astype(np.float32) for _ in range(3))
    m = oracle.run(q, k, v, g, precision="mix")
    b = oracle.run(q, k, v, g)
    # Selection uses unquantised Q/K: identical lists.
    assert np.array_equal(m["select_idx"], b["select_idx"])
    p = m["plan"]
    qd = np.empty_like(m["qp"], dtype=np.float64)
    kd = np.empty_like(m["kp"], dtype=np.float64)
    for j, (r0, n) in enumerate(p.blocks):
        qd[:, :, r0:r0 + n] = e4m3_decode(m["q8"][:, :, r0:r0 + n]) * m["q_scale"][:, :, j, None, None]
        kd[:, :, r0:r0 + n] = e4m3_decode(m["k8"][:, :, r0:r0 + n]) * m["k_scale"][:, :, j, None, None]
    ref = oracle.sparse_attention(qd, kd, m["vp"], p, m["select_idx"], m["select_num"], m["scale"])
    np.testing.assert_allclose(m["out_p"], ref, rtol=0, atol=1e-13)
    # Quantisation moves the output only a little.
    assert np.abs(m["out"] - b["out"]).max() < 6e-2
