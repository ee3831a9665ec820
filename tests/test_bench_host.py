"""Host logic of bench.py: the flop accounting, the traffic gate and the one-GPU refusal.

The attention flops that bench.py reports are Σ over query rows × listed key
rows × 4·D. The key rows come from the plan's block table. They are checked
here against the oracle's block table ("RainFusion Attention", Geometry
handling: ceiling division for the ragged head and tail segments) and against
hand-made lists.
"""
import hashlib
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import block_sparse_video_rf_amd as rf
from oracle.geometry import plan
from synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

from gpu_harness import geometry_of  # noqa: E402


@pytest.mark.parametrize("name", ["tiny", "wan22", "minimax_h3", "gqa_long"])
def test_block_lengths_match_oracle_table(name):
    w = WORKLOADS[name]
    desc = rf.Desc.from_workload(w)
    info = rf.rf_plan(desc)
    p = plan(geometry_of(desc))
    want = np.array([n for _, n in p.blocks], dtype=np.int64)
    got = bench._block_lengths(info)
    assert np.array_equal(got, want)
    assert got.sum() == desc.seq_len


def test_listed_key_rows_hand_made():
    lengths = np.array([128, 100, 32], dtype=np.int64)
    idx = np.array([[[0, 2, -1], [1, -1, -1]],
                    [[0, 1, 2], [2, 0, 1]]], dtype=np.int32)
    num = np.array([[2, 1], [3, 1]], dtype=np.int32)
    got = bench.listed_key_rows(idx, num, lengths)
    # Entries past selectNum and -1 entries count nothing.
    assert got.tolist() == [[160, 100], [260, 32]]


@pytest.mark.parametrize("workload", ["wan22", "wan22_mix", "wan22_fp8", "wan22_mxfp4"])
def test_traffic_needs_the_profiled_kernel_source(tmp_path, monkeypatch, workload):
    path = bench.traffic_file(workload)
    if not os.path.exists(path):
        pytest.skip("no counter summary committed for " + workload)
    vals = {k.strip(): v.strip() for k, v in
            (line.split(":", 1) for line in open(path) if ":" in line)}
    current = hashlib.sha256(open(bench.ATTN_SRC, "rb").read()).hexdigest()
    got = bench.traffic_from_profile(workload)
    if vals.get("source_sha256") == current:
        assert got == pytest.approx(float(vals["traffic_bytes_per_launch"]))
    else:
        assert got is None
    src = tmp_path / "rf_attn.hip"
    shutil.copy(bench.ATTN_SRC, src)
    with open(src, "a") as f:
        f.write("\n// changed\n")
    monkeypatch.setattr(bench, "ATTN_SRC", str(src))
    assert bench.traffic_from_profile(workload) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
