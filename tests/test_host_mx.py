"""The kernels' MXFP4 block-exponent rule (rf_mx_scale_exp, used by the permute
kernel for Q/K/V and by the attention kernel for P) compiled for the host and
compared with the oracle's UOS exponent on every kind of float32 block maximum.
No GPU needed."""
import os
import subprocess

import numpy as np
import pytest

from oracle.mxfp4 import mx_scale_exponent

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def dump_exe(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("mx") / "mx_exp_dump")
    subprocess.run(["g++", "-O1", "-std=c++17", "-fsanitize=address,undefined",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "block_sparse_video_rf_amd", "csrc"),
                    os.path.join(HERE, "host", "mx_exp_dump.cpp"), "-o", exe], check=True)
    return exe


def _run(exe, tmp_path, x):
    x = np.asarray(x, dtype=np.float32)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    x.tofile(src)
    subprocess.run([exe, str(src), str(dst)], check=True)
    return np.fromfile(dst, dtype=np.int32)


def test_exponent_rule_matches_oracle(dump_exe, tmp_path):
    edges = []
    for k in range(-135, 126):                      # 7.25 * 2^k as float32 (exact when normal)
        e = np.float32(7.25 * 2.0 ** k)
        if e > 0:
            edges += [e, np.nextafter(e, np.float32(np.inf)), np.nextafter(e, np.float32(0))]
    special = [0.0, np.float32(2.0 ** -149), np.float32(2.0 ** -126), np.nextafter(np.float32(2.0 ** -126), 0),
               np.float32(3.0e38), np.finfo(np.float32).max, 1.0, 1.8125, 1.8125001, 6.0, 7.0, 8.0]
    rng = np.random.default_rng(21)
    bits = rng.integers(0, 0x7F800000, 200000, dtype=np.int64).astype(np.uint32)   # every finite >= 0
    rand = bits.view(np.float32)
    x = np.concatenate([np.array(edges, dtype=np.float32), np.array(special, dtype=np.float32), rand])
    got = _run(dump_exe, tmp_path, x)
    want = mx_scale_exponent(x.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(want[i])) for i in bad[:5]]
    # The boundary itself: 7.25 * 2^k maps to k, the next float above to k + 1.
    assert _run(dump_exe, tmp_path, [7.25, np.nextafter(np.float32(7.25), np.float32(8))]).tolist() == [0, 1]
