"""E4M3 codes of every bf16 value: the permute's quantisation against the oracle's encoder.

Channel 0 of every row holds 448, so every block's absolute maximum is 448.
The mix scale 448 / amax is then exactly 1, and so is the fp8 power-of-two V scale.
The codes are then the E4M3 encodings of the bf16 values themselves.
The other channels run through every finite bf16 value of magnitude <= 448 in both signs:
- the ties of the 3-bit mantissa;
- the E4M3 subnormals;
- values that round to zero;
- zeros of both signs.
The codes must be bit-identical to the oracle's round-to-nearest-even encoder
("RainFusion Attention", Wan2.2 T2V quantization; the OCP FP8 E4M3 format).
"""
import numpy as np
import pytest

import oracle
from oracle.geometry import permutation, plan
from synth import WORKLOADS

from gpu_harness import expected_vpt, geometry_of, log, to_dev

pytestmark = pytest.mark.gpu

MAX_BF16 = 0x43E0  # 448.0


def sweep_inputs(heads, S, D):
    """bf16 bit patterns [1, heads, S, D]: 448 in channel 0, every |x| <= 448 elsewhere."""
    pos = np.arange(MAX_BF16 + 1, dtype=np.uint16)
    vals = np.concatenate([pos, pos | np.uint16(0x8000)])
    n = heads * S * (D - 1)
    body = np.resize(vals, n).reshape(1, heads, S, D - 1)
    x = np.empty((1, heads, S, D), dtype=np.uint16)
    x[..., 0] = MAX_BF16
    x[..., 1:] = body
    return x, vals.size


@pytest.mark.parametrize("precision", ["mix", "fp8"])
def test_codes_of_every_bf16_value(precision):
    import torch
    import block_sparse_video_rf_amd as rf
    w = WORKLOADS["tiny"].with_(head_dim=128, precision=precision)
    desc = rf.Desc.from_workload(w)
    g = geometry_of(desc)
    p = plan(g)
    pi = permutation(g)
    S, D = desc.seq_len, w.head_dim
    x, nvals = sweep_inputs(w.heads_q, S, D)
    assert x.size > 2 * nvals  # every value appears in Q, K and V alike
    log(f"[codes {precision}] S={S} D={D} values={nvals}")
    q = to_dev(x)
    bufs = rf.Buffers(desc, device=q.device)
    b = bufs
    rf.rf_permute(desc, q, q, q, b.qp, b.kp, b.vpt, b.q_pool, b.k_pool, b.q8, b.k8, b.q_scale,
                  b.k_scale, b.v_scale)
    torch.cuda.synchronize()

    xf = oracle.permute_rows(x, pi)
    xf = (xf.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    codes, scales = oracle.quantize_blocks(xf, p)
    assert np.all(scales == 1.0)
    assert np.array_equal(b.q8.cpu().numpy(), codes)
    assert np.array_equal(b.k8.cpu().numpy(), codes)
    assert np.array_equal(b.q_scale.cpu().numpy(), scales)
    if precision == "fp8":
        v8, sv = oracle.quantize_blocks_pow2(xf, p)
        assert np.all(sv == 1.0)
        assert np.array_equal(b.vpt.cpu().numpy(), expected_vpt(v8, p, D))
        assert np.array_equal(b.v_scale.cpu().numpy(), sv)
