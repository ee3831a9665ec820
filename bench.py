#!/usr/bin/env python3
"""Benchmark of the block-sparse video attention path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
rf_permute -> rf_pool_select -> rf_sparse_attn -> rf_unpermute, with the
inputs already resident in HBM. The default workload is the Wan2.2-style
720p latent grid (B=1, 40 heads, D=128, 512-row prefix + grid (21, 40, 64),
sparsity 0.8, bf16).

Printed (one JSON line): the sparse attention kernel's ms/call (``value``),
its actual and dense-equivalent TFLOP/s and MFMA-roofline fraction, the
pipeline ms/step, the same kernel run with every block listed (dense), the
dense path (rf_dense_attn) and the speed-up against the ceiling set by the
always-dense rows, per-kernel times of
the bandwidth-bound steps, and the CPU oracle timed on a bounded sample.

Kernel times come from HIP events recorded on the stream the library
launches on (torch's current stream, passed to every rf_* call).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse attn ms/call + dense-equiv TFLOPS & MFMA util at 0.8 sparsity, 1 MI355X"
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}
HBM_PEAK_GBS = 8000.0
ATTN_SRC = os.path.join(ROOT, "block_sparse_video_rf_amd", "csrc", "rf_attn.hip")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan22")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (profiling runs)")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense comparison run")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure the achievable peaks: an MFMA microbenchmark (bf16, fp8), an LDS / VALU microbenchmark, "
                         "a large bf16 GEMM (hipBLASLt) and a "
                         "device-to-device copy")
    return ap.parse_args()


def measure_peaks(torch, dev):
    """Achievable MFMA and HBM rates on this machine, to read the rooflines against."""
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.mm(a, b, out=c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        torch.mm(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    gemm_ms = e0.elapsed_time(e1) / reps
    x = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    for _ in range(2):
        y.copy_(x)
    e0.record()
    for _ in range(5):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / 5
    # Matrix-core rate with operands in registers (tests/native/mfma_peak, built
    # by __graft_entry__.build()).
    mfma = None
    exe = os.path.join(ROOT, "tests", "native", "mfma_peak")
    if os.path.exists(exe):
        import subprocess
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        if r.returncode == 0:
            m = json.loads(r.stdout.strip().splitlines()[-1])
            mfma = {"bf16_tflops": m["mfma_bf16_tflops"],
                    "bf16_frac_of_published": round(m["mfma_bf16_tflops"] / PEAK_TFLOPS["bf16"], 3),
                    "fp8_tflops": m["mfma_fp8_tflops"],
                    "fp8_frac_of_published": round(m["mfma_fp8_tflops"] / PEAK_TFLOPS["fp8"], 3)}
    # LDS bandwidth and vector-ALU issue costs in shader cycles
    # (tests/native/lds_valu_peak).
    lds_valu = None
    exe = os.path.join(ROOT, "tests", "native", "lds_valu_peak")
    if os.path.exists(exe):
        import subprocess
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        if r.returncode == 0:
            lds_valu = json.loads(r.stdout.strip().splitlines()[-1])
    return {"mfma_microbenchmark": mfma, "lds_valu_microbenchmark": lds_valu,
            "gemm_bf16": {"m": n, "n": n, "k": n, "ms": round(gemm_ms, 4),
                          "tflops": round(2.0 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
                          "frac_of_published": round(2.0 * n ** 3 / (gemm_ms * 1e-3) / 1e12
                                                     / PEAK_TFLOPS["bf16"], 3)},
            "copy": {"bytes_moved": 2 * (1 << 32), "ms": round(copy_ms, 4),
                     "GB_s": round(2 * (1 << 32) / (copy_ms * 1e-3) / 1e9, 1),
                     "frac_of_published": round(2 * (1 << 32) / (copy_ms * 1e-3) / 1e9
                                                / HBM_PEAK_GBS, 3)}}


def _block_lengths(info):
    """Row count of every block id (host copy of the plan's block table)."""
    L = np.full(info.n_blocks, 128, dtype=np.int64)
    if info.n_head:
        L[info.n_head - 1] = info.head_rows - 128 * (info.n_head - 1)
    if info.n_tail:
        L[-1] = info.promoted_rows - 128 * (info.n_tail - 1)
    return L


def listed_key_rows(select_idx, select_num, lengths):
    """Per selectIdx row and head: the number of key rows listed."""
    idx = select_idx.astype(np.int64)
    valid = (np.arange(idx.shape[-1])[None, None, :] < select_num[:, :, None]) & (idx >= 0)
    return np.where(valid, lengths[np.clip(idx, 0, None)], 0).sum(axis=-1)


def traffic_file(workload):
    """The committed counter summary of the attention kernel on this workload."""
    return os.path.join(ROOT, "profiles", f"sparse_attn_kernel_{workload}_pmc.txt")


def traffic_from_profile(workload):
    """HBM bytes per launch of the attention kernel from the committed counter summary
    of this workload, or None when it is absent or was taken on a different kernel
    source."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    want = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != want:
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


HBM_STEP_SOURCES = {
    "permute": os.path.join(ROOT, "block_sparse_video_rf_amd", "csrc", "rf_permute.hip"),
    "unpermute": os.path.join(ROOT, "block_sparse_video_rf_amd", "csrc", "rf_permute.hip"),
    "score": os.path.join(ROOT, "block_sparse_video_rf_amd", "csrc", "rf_select.hip"),
    "select": os.path.join(ROOT, "block_sparse_video_rf_amd", "csrc", "rf_select.hip"),
}


def hbm_counters_from_profile(workload):
    """HBM bytes per launch of the bandwidth-bound kernels (FETCH_SIZE +
    WRITE_SIZE, calibrated) from the committed counter summary of this workload,
    per step, for the steps whose kernel source is unchanged since; {} if none."""
    path = os.path.join(ROOT, "profiles", f"hbm_steps_{workload}_pmc.txt")
    if not os.path.exists(path):
        return {}
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    out = {}
    for step, src in HBM_STEP_SOURCES.items():
        key = f"{step}_bytes_per_launch"
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if key in vals and vals.get(f"source_sha256_{os.path.basename(src)}") == sha:
            out[step] = {"bytes": float(vals[key]),
                         "kernel_ms": float(vals.get(f"{step}_kernel_ms", "nan"))}
    return out


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, q, k, v, gi, gn, lengths, target_s):
    """Time the oracle (as it stands) on a bounded sample and scale to ms per call."""
    import oracle
    from oracle.geometry import Geometry, permutation, plan
    from synth import bf16_to_f32
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    g = Geometry(w.prefix_len, w.grid, w.first_frame, w.sparsity)
    p = plan(g)
    scale = 1.0 / math.sqrt(w.head_dim)
    G = w.heads_q // w.heads_kv
    t0 = time.perf_counter()
    pi = permutation(g)
    # Selection steps on the first two heads (per-head work; scaled by heads / 2).
    hs = min(2, w.heads_q)
    qp = bf16_to_f32(oracle.permute_rows(q[:, :hs], pi))
    kp = bf16_to_f32(oracle.permute_rows(k[:, :max(1, hs // G)], pi))
    qb, kb = oracle.pool_blocks(qp, p), oracle.pool_blocks(kp, p)
    sc = oracle.block_scores(qb, kb, scale)
    oracle.select_lists(p, 1, hs, sc)
    t_sel = (time.perf_counter() - t0) * (w.heads_q / hs)
    # Attention on sampled (query block, head) pairs, stratified dense / sparse.
    rng = np.random.default_rng(5)
    nB = p.n_blocks
    dense_q = [qq for qq in range(nB) if not p.is_sparse_block(qq)]
    sparse_q = [qq for qq in range(nB) if p.is_sparse_block(qq)]
    kpf_cache = {}
    done = {"dense": [0, 0.0], "sparse": [0, 0.0]}
    t_start = time.perf_counter()
    while time.perf_counter() - t_start < target_s:
        for kind, pool in (("dense", dense_q), ("sparse", sparse_q)):
            if not pool:
                continue
            qq = int(rng.choice(pool))
            n = int(rng.integers(w.heads_q))
            nk = n // G
            if nk not in kpf_cache:
                kpf_cache[nk] = (bf16_to_f32(oracle.permute_rows(k[0, nk], pi, axis=0)),
                                 bf16_to_f32(oracle.permute_rows(v[0, nk], pi, axis=0)))
            kf, vf = kpf_cache[nk]
            a = time.perf_counter()
            r0, m = p.blocks[qq]
            qrows = bf16_to_f32(q[0, n, pi[r0:r0 + m]])
            ids = gi[qq, n, :gn[qq, n]]
            rows = oracle.attention.listed_rows(p, ids)
            oracle.attention_block(qrows, kf[rows], vf[rows], scale)
            done[kind][0] += 1
            done[kind][1] += time.perf_counter() - a
    n_dense_units = len(dense_q) * w.heads_q * w.batch
    n_sparse_units = len(sparse_q) * w.heads_q * w.batch
    t_attn = 0.0
    for kind, units in (("dense", n_dense_units), ("sparse", n_sparse_units)):
        if done[kind][0]:
            t_attn += done[kind][1] / done[kind][0] * units
    return {
        "value": round(t_attn * 1e3, 1), "unit": "ms/call", "cores": int(cores),
        "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
        "sample": (f"float64 NumPy oracle: attention on {done['dense'][0]} dense + "
                   f"{done['sparse'][0]} sparse sampled (query block, head) pairs of the "
                   f"{w.name} workload (of {n_dense_units} + {n_sparse_units}), scaled by the "
                   f"pair counts; selection (pool, score, top-k) on {hs} of {w.heads_q} heads "
                   f"took {t_sel:.1f} s scaled to all heads"),
        "selection_s": round(t_sel, 2),
    }


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: the path runs on one GPU; --gpus {args.gpus} is not supported "
              "(a multi-GPU version would shard it by head, which is not implemented)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import block_sparse_video_rf_amd as rf
    from synth import get_workload, make_qkv

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.peaks:
        print(json.dumps({"peaks_measured": measure_peaks(torch, dev)}))
        return

    if args.copy_calibration:
        x = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "launches": 3}))
        return

    w = get_workload(args.workload)
    desc = rf.Desc.from_workload(w)
    info = rf.rf_plan(desc)
    t0 = time.perf_counter()
    qh, kh, vh = make_qkv(w)
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    q, k, v = to_dev(qh), to_dev(kh), to_dev(vh)
    out = torch.empty_like(q)
    bufs = rf.Buffers(desc, device=dev)
    gen_s = time.perf_counter() - t0
    nB = info.n_blocks
    stream = torch.cuda.current_stream()

    def step(ev=None):
        b = bufs
        if ev is not None:
            ev[0].record(stream)
        rf.rf_permute(desc, q, k, v, b.qp, b.kp, b.vpt, b.q_pool, b.k_pool, b.q8, b.k8,
                      b.q_scale, b.k_scale, b.v_scale, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        rf.rf_pool_select(desc, b.qp, b.kp, b.q_pool, b.k_pool, b.select_idx, b.select_num, nB,
                          b.workspace, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        rf.rf_sparse_attn(desc, b.qp, b.kp, b.vpt, b.q8, b.k8, b.q_scale, b.k_scale, b.v_scale,
                          b.select_idx, b.select_num, nB, b.out_p, stream=stream)
        if ev is not None:
            ev[3].record(stream)
        rf.rf_unpermute(desc, b.out_p, out, stream=stream)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_start) * 1e3 / args.steps
    seg = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in evs])  # ms
    step_ms = np.array([e[0].elapsed_time(e[4]) for e in evs])
    permute_ms, select_ms, attn_ms, unpermute_ms = (float(np.mean(seg[:, i])) for i in range(4))
    attn_med = float(np.median(seg[:, 2]))

    # Algorithmic work from the lists actually used.
    gi = bufs.select_idx.cpu().numpy()
    gn = bufs.select_num.cpu().numpy()
    L = _block_lengths(info)
    qlen = np.tile(L, w.batch)[:, None]                  # query rows of each selectIdx row
    pairs = float((listed_key_rows(gi, gn, L) * qlen).sum())
    flops = 4.0 * w.head_dim * pairs
    dense_flops = 4.0 * w.head_dim * w.heads_q * w.batch * float(w.seq_len) ** 2
    tflops = flops / (attn_ms * 1e-3) / 1e12
    tflops_dense_eq = dense_flops / (attn_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS["bf16"]
    if w.precision == "mix":
        peak = 2.0 / (1.0 / PEAK_TFLOPS["fp8"] + 1.0 / PEAK_TFLOPS["bf16"])  # QK^T fp8, PV bf16
    elif w.precision == "fp8":
        peak = PEAK_TFLOPS["fp8"]                                            # both products fp8
    elif w.precision == "mxfp4":
        peak = PEAK_TFLOPS["fp4"]                                            # both products fp4
    ceiling = dense_flops / flops

    dense = None
    if not args.no_dense:
        idx_d = torch.arange(nB, dtype=torch.int32, device=dev).expand(
            w.batch * nB, w.heads_q, nB).contiguous()
        num_d = torch.full((w.batch * nB, w.heads_q), nB, dtype=torch.int32, device=dev)
        out_d = torch.empty_like(bufs.out_p)
        b = bufs
        for _ in range(2):
            rf.rf_sparse_attn(desc, b.qp, b.kp, b.vpt, b.q8, b.k8, b.q_scale, b.k_scale,
                              b.v_scale, idx_d, num_d, nB, out_d, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(3, args.steps // 4)
        e0.record(stream)
        for _ in range(reps):
            rf.rf_sparse_attn(desc, b.qp, b.kp, b.vpt, b.q8, b.k8, b.q_scale, b.k_scale,
                              b.v_scale, idx_d, num_d, nB, out_d, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / reps
        # The dense path proper (rf_dense_attn: same kernel, no lists to read).
        e0.record(stream)
        for _ in range(reps):
            rf.rf_dense_attn(desc, b.qp, b.kp, b.vpt, b.q8, b.k8, b.q_scale, b.k_scale,
                             b.v_scale, out_d, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_path_ms = e0.elapsed_time(e1) / reps
        # The ceiling is the flop ratio the always-dense rows leave (prefix, first
        # frame and promoted rows attend to every block): the speed-up of a
        # kernel with the same per-flop rate on both runs.
        dense = {"ms_per_call": round(dense_ms, 3), "speedup": round(dense_ms / attn_ms, 3),
                 "speedup_ceiling": round(ceiling, 3),
                 "speedup_frac_of_ceiling": round(dense_ms / attn_ms / ceiling, 3),
                 "speedup_target": 3.5,
                 "target_within_ceiling": bool(ceiling >= 3.5),
                 "tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 1),
                 "dense_path_ms": round(dense_path_ms, 3),
                 "dense_path_tflops": round(dense_flops / (dense_path_ms * 1e-3) / 1e12, 1)}
        del idx_d, num_d, out_d

    S, D, N1, N2, B = w.seq_len, w.head_dim, w.heads_q, w.heads_kv, w.batch
    # permute: read Q, K, V once; write the permuted Q/K (bf16, or E4M3 codes in mix
    # and fp8, E2M1 codes plus one E8M0 byte per 32 in mxfp4), the block-transposed V
    # (blocks padded to 128 columns; E4M3 in fp8, E2M1 plus scales in mxfp4) and the
    # pooled means.
    qk_out = {"bf16": 2.0, "mix": 1.0, "fp8": 1.0, "mxfp4": 0.5 + 1.0 / 32}[w.precision]
    v_out = {"bf16": 2.0, "mix": 2.0, "fp8": 1.0, "mxfp4": 0.5 + 1.0 / 32}[w.precision]
    perm_bytes = (2.0 * S * D * B * (N1 + 2 * N2) + qk_out * S * D * B * (N1 + N2)
                  + v_out * nB * 128 * D * B * N2 + 4.0 * info.n_sparse * D * B * (N1 + N2))
    unperm_bytes = 4.0 * S * D * B * N1
    hbm = {
        "permute": {"ms": round(permute_ms, 4), "bytes": perm_bytes,
                    "GB_s": round(perm_bytes / permute_ms / 1e6, 1)},
        "pool_select": {"ms": round(select_ms, 4)},
        "unpermute": {"ms": round(unpermute_ms, 4), "bytes": unperm_bytes,
                      "GB_s": round(unperm_bytes / unpermute_ms / 1e6, 1)},
        "peak_GB_s": HBM_PEAK_GBS,
    }
    # Counter-measured HBM bytes (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated
    # on a plain copy) from the committed summary, over this run's times: the
    # rate each step actually drew from HBM, against the 8 TB/s peak.
    counters = hbm_counters_from_profile(w.name)
    for step_name, ms in (("permute", permute_ms), ("unpermute", unpermute_ms)):
        if step_name in counters:
            cb = counters[step_name]["bytes"]
            hbm[step_name].update(counter_bytes=cb, counter_GB_s=round(cb / ms / 1e6, 1),
                                  counter_frac_of_peak=round(cb / ms / 1e6 / HBM_PEAK_GBS, 3))
    if "score" in counters and "select" in counters:
        cb = counters["score"]["bytes"] + counters["select"]["bytes"]
        hbm["pool_select"].update(counter_bytes=cb, counter_GB_s=round(cb / select_ms / 1e6, 1),
                                  counter_frac_of_peak=round(cb / select_ms / 1e6 / HBM_PEAK_GBS, 3))

    traffic = traffic_from_profile(args.workload)
    result = {
        "metric": METRIC,
        "value": round(attn_ms, 4),
        "unit": "ms/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(float(np.mean(step_ms)), 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "mix": "fp8e4m3-qk/bf16-pv", "fp8": "fp8e4m3",
                  "mxfp4": "mxfp4"}[w.precision],
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "heads_q": N1, "heads_kv": N2, "head_dim": D,
                   "seq_len": S, "prefix_len": w.prefix_len, "grid": list(w.grid),
                   "first_frame_rows": w.first_frame_rows, "sparsity": w.sparsity,
                   "precision": w.precision, "layout": "BNSD", "block": [128, 128]},
        "attn_ms_median": round(attn_med, 4),
        "attn_tflops": round(tflops, 1),
        "attn_dense_equiv_tflops": round(tflops_dense_eq, 1),
        "mfma_util": round(tflops / peak, 4),
        "attn_flops_per_call": flops,
        "dense": dense,
        "hbm_steps": hbm,
        "wall_ms_per_step": round(wall_ms, 4),
        "input_gen_s": round(gen_s, 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": round(peak, 1),
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                     "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, qh, kh, vh, gi, gn, L, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
