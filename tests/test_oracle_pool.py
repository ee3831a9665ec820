"""The process pool that spreads the oracle over (query block, head) pairs
for the full-size GPU checks (tests/oracle_pool.py), on the CPU: fed the
oracle's own output, every pair passes in each mode; an error planted in one
pair's output fails exactly that pair."""
import numpy as np

import oracle
from oracle.geometry import Geometry, plan
from synth import WORKLOADS, bf16_to_f32, make_qkv

from oracle_pool import compare_pairs


def _dequant(codes, sigma, p):
    d = np.empty(codes.shape)
    for j, (r0, n) in enumerate(p.blocks):
        d[:, :, r0:r0 + n] = oracle.e4m3_decode(codes[:, :, r0:r0 + n]) * sigma[:, :, j, None, None]
    return d


def test_pool_modes_and_a_planted_error():
    w = WORKLOADS["tiny"]
    g = Geometry(w.prefix_len, w.grid, True, w.sparsity)
    p = plan(g)
    q, k, v = (bf16_to_f32(x) for x in make_qkv(w))
    scale = 1.0 / np.sqrt(w.head_dim)
    pairs = [(0, qb, n) for qb in (0, 3, 10, 20, 36) for n in range(w.heads_q)]
    for mode in ("bf16", "mix", "fp8"):
        res = oracle.run(q, k, v, g, precision="bf16" if mode == "bf16" else mode)
        lists = (res["select_idx"], res["select_num"])
        out = res["out_p"].astype(np.float32)
        arrays = dict(out=out, q=res["qp"], k=res["kp"], v=res["vp"])
        if mode != "bf16":
            arrays.update(qd=_dequant(res["q8"], res["q_scale"], p),
                          kd=_dequant(res["k8"], res["k_scale"], p))
        if mode == "fp8":
            arrays["vd"] = _dequant(res["v8"], res["v_scale"], p)
        kw = dict(tol=(2e-2, 2e-3), kernel_tol=(2e-2, 2e-3))
        if mode == "mix":
            kw["tol"] = (6e-2, 6e-3)
        got = compare_pairs(arrays, p.blocks, pairs, lists, scale, 1, mode, workers=2, **kw)
        assert len(got) == len(pairs) and all(r["ok"] for r in got), mode
        r0, m = p.blocks[10]
        out[0, 1, r0 + 5, 7] += 0.5
        got = compare_pairs(arrays | {"out": out}, p.blocks, pairs, lists, scale, 1, mode,
                            workers=2, **kw)
        bad = [r["pair"] for r in got if not r["ok"]]
        assert bad == [(0, 10, 1)], (mode, bad)
