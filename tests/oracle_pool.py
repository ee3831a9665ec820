"""The oracle's attention on many (batch, query block, head) pairs at once, in
worker processes (test infrastructure).

Full-size parity needs the float64 oracle on thousands of (query block, head)
pairs. Each pair is ``oracle.attention_block`` (or the quantised readings) on
the listed key rows, exactly as ``oracle.sparse_attention`` evaluates it; this
module only spreads the pairs over processes. Workers are started with
``spawn`` and import numpy and ``oracle`` alone (never torch or the HIP
library); they read the operands and the GPU's output through memory-mapped
``.npy`` files and send back error statistics per pair, not outputs.

Comparison per pair (``mode``):
* ``bf16``: the GPU against the exact oracle, max-abs and mean-abs within
  ``tol`` (the bf16 bound);
* ``mix``: the GPU against the oracle on dequantised Q/K (``kernel_tol``), and
  against the exact oracle within the mix bound, or within the quantised
  reading's own deviation plus ``kernel_tol`` where that is larger;
* ``fp8``, ``mxfp4``: the GPU against the fp8 (mxfp4) reading on the same
  codes within the derived per-element bound (tests/fp8_bounds.py), and
  against the exact oracle within the reading's own deviation plus that
  bound.
"""
from __future__ import annotations

import os
import tempfile
import types
from concurrent.futures import ProcessPoolExecutor
from multiprocessing import get_context

import numpy as np

_W = {}


def _init(paths, blocks, scale, G, mode, tol, kernel_tol):
    _W.update({k: np.load(v, mmap_mode="r") for k, v in paths.items()})
    _W.update(blocks=blocks, scale=scale, G=G, mode=mode, tol=tol, kernel_tol=kernel_tol)


def _rows(ids):
    blocks = _W["blocks"]
    parts = [np.arange(blocks[j][0], blocks[j][0] + blocks[j][1]) for j in ids]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def _pair(b, q, n, ids):
    import oracle
    from fp8_bounds import kernel_bound, mx_kernel_bound
    W = _W
    r0, m = W["blocks"][q]
    G, scale, mode = W["G"], W["scale"], W["mode"]
    rows = _rows(ids)
    got = np.asarray(W["out"][b, n, r0:r0 + m], np.float64)
    exact = oracle.attention_block(W["q"][b, n, r0:r0 + m], W["k"][b, n // G, rows],
                                   W["v"][b, n // G, rows], scale)
    err = np.abs(got - exact)
    res = {"pair": (b, q, n), "max": float(err.max()), "sum": float(err.sum()), "n": err.size}
    if mode == "bf16":
        res["ok"] = bool(err.max() <= W["tol"][0] and err.mean() <= W["tol"][1])
        return res
    qd, kd = W["qd"][b, n, r0:r0 + m], W["kd"][b, n // G, rows]
    if mode == "mix":
        reading = oracle.attention_block(qd, kd, W["v"][b, n // G, rows], scale)
        e_same = np.abs(got - reading)
        own = np.abs(reading - exact)
        kt, tol = W["kernel_tol"], W["tol"]
        res.update(same_max=float(e_same.max()), same_sum=float(e_same.sum()),
                   own_max=float(own.max()))
        res["ok"] = bool(e_same.max() <= kt[0] and e_same.mean() <= kt[1]
                         and err.max() <= max(tol[0], own.max() + kt[0])
                         and err.mean() <= max(tol[1], own.mean() + kt[1]))
        return res
    vd = W["vd"][b, n // G, rows]
    groups = oracle.attention.listed_groups(types.SimpleNamespace(blocks=W["blocks"]), ids)
    if mode == "mxfp4":
        reading = oracle.attention_block_mxp(qd, kd, vd, scale, groups)
        bound = mx_kernel_bound(qd, kd, vd, scale, groups)
    else:
        reading = oracle.attention_block_fp8p(qd, kd, vd, scale)
        bound = kernel_bound(qd, kd, vd, scale, groups)
    e_same = np.abs(got - reading)
    own = np.abs(reading - exact)
    res.update(same_max=float(e_same.max()), same_sum=float(e_same.sum()),
               ratio=float((e_same / bound).max()), own_max=float(own.max()))
    res["ok"] = bool(np.all(e_same <= bound) and np.all(err <= own + bound))
    return res


def _chunk(tasks):
    return [_pair(*t) for t in tasks]


def compare_pairs(arrays, blocks, pairs, lists, scale, G, mode, tol=None, kernel_tol=None,
                  workers=None, chunk=8):
    """Compare the GPU output with the oracle on ``pairs`` [(b, q, n)].

    ``arrays``: ``out`` (GPU output, permuted rows, float32 ``[B, N1, S, D]``),
    ``q``, ``k``, ``v`` (permuted inputs), and for ``mix`` ``qd``, ``kd``
    (dequantised Q/K), for ``fp8`` and ``mxfp4`` also ``vd``. ``lists``: (select_idx,
    select_num). Returns the per-pair results (dicts with ``ok``)."""
    idx, num = lists
    nB = len(blocks)
    tasks = [(b, q, n, np.asarray(idx[b * nB + q, n, :num[b * nB + q, n]]).tolist())
             for b, q, n in pairs]
    workers = workers or max(1, min(16, os.cpu_count() or 1))
    with tempfile.TemporaryDirectory(prefix="oracle_pool_") as d:
        paths = {}
        for name, a in arrays.items():
            paths[name] = os.path.join(d, name + ".npy")
            np.save(paths[name], np.ascontiguousarray(a))
        here = os.path.dirname(os.path.abspath(__file__))
        root = os.path.dirname(here)
        # Workers inherit the environment: the tests and the repository on the
        # path, and one BLAS thread each (the pairs are the parallelism).
        saved = {k: os.environ.get(k) for k in ("PYTHONPATH", "OMP_NUM_THREADS",
                                                "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
        os.environ["PYTHONPATH"] = os.pathsep.join(
            x for x in (here, root, saved["PYTHONPATH"] or "") if x)
        for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
            os.environ[k] = "1"
        try:
            with ProcessPoolExecutor(max_workers=workers, mp_context=get_context("spawn"),
                                     initializer=_init,
                                     initargs=(paths, list(blocks), scale, G, mode, tol,
                                               kernel_tol)) as ex:
                chunks = [tasks[i:i + chunk] for i in range(0, len(tasks), chunk)]
                out = []
                for r in ex.map(_chunk, chunks):
                    out.extend(r)
        finally:
            for k, val in saved.items():
                if val is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = val
    return out
