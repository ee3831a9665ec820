"""The library's index math (rf_natural_row, rf_block_rows, as the kernels use
them) compiled for the host and compared with the oracle's permutation and
block table on many geometries, bit for bit. No GPU needed."""
import os
import subprocess

import numpy as np
import pytest

from oracle.geometry import Geometry, permutation, plan

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def dump_exe(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("geom") / "geometry_dump")
    srcs = [os.path.join(HERE, "host", "geometry_dump.cpp"),
            os.path.join(ROOT, "block_sparse_video_rf_amd", "csrc", "rf_api.cpp")]
    # rf_api.cpp refers to the launchers; stub them for this host-only program.
    stub = str(tmp_path_factory.mktemp("stub") / "stub.cpp")
    with open(stub, "w") as f:
        f.write('#include "rf_internal.h"\n'
                'rf_status rf_launch_permute(const RfGeom&, int32_t, const void*, const void*, '
                'const void*, void*, void*, void*, float*, float*, uint8_t*, uint8_t*, void*, '
                'void*, void*, void*) { return RF_ERR_HIP; }\n'
                'rf_status rf_launch_unpermute(const RfGeom&, const void*, void*, void*) '
                '{ return RF_ERR_HIP; }\n'
                'rf_status rf_launch_pool_select(const RfGeom&, float, const void*, const void*, '
                'const float*, const float*, int32_t*, int32_t*, int32_t, void*, void*) '
                '{ return RF_ERR_HIP; }\n'
                'rf_status rf_noalloc_scratch(void**) { return RF_ERR_HIP; }\n'
                'rf_status rf_launch_sparse_attn(const RfGeom&, int32_t, float, const void*, '
                'const void*, const void*, const uint8_t*, const uint8_t*, const void*, '
                'const void*, const void*, const int32_t*, const int32_t*, int32_t, void*, '
                'void*) '
                '{ return RF_ERR_HIP; }\n')
    subprocess.run(["g++", "-O1", "-std=c++17", "-fsanitize=address,undefined",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "block_sparse_video_rf_amd", "csrc"),
                    *srcs, stub, "-o", exe], check=True)
    return exe


GEOMS = [(128, (9, 16, 32), 1, 0.8, 32), (512, (62, 24, 42), 0, 0.8, 32),
         (200, (10, 17, 34), 1, 0.8, 32), (512, (6, 24, 42), 0, 0.8, 1),
         (77, (5, 16, 40), 1, 0.5, 32), (128, (3, 8, 248), 1, 0.8, 32),
         (128, (3, 8, 256), 1, 0.8, 32), (0, (4, 16, 16), 0, 1.0, 1),
         (300, (8, 11, 17), 1, 0.8, 1), (64, (7, 9, 9), 1, 0.3, 1), (33, (2, 8, 8), 0, 0.8, 1),
         (1000, (1, 1, 1), 0, 0.8, 32), (512, (21, 40, 64), 1, 0.8, 32),
         (5, (11, 23, 15), 0, 0.9, 1), (129, (6, 15, 49), 1, 0.7, 1)]


@pytest.mark.parametrize("P,grid,f0,s,mb", GEOMS)
def test_index_math_matches_oracle(dump_exe, P, grid, f0, s, mb):
    out = subprocess.run([dump_exe, str(P), *map(str, grid), str(f0), str(s), str(mb)],
                         check=True, capture_output=True, text=True).stdout.split("\n")
    S = int(out[0])
    pi = np.array(out[1:1 + S], dtype=np.int64)
    nb = int(out[1 + S])
    blocks = [tuple(map(int, line.split())) for line in out[2 + S:2 + S + nb]]
    g = Geometry(P, grid, bool(f0), s, min_sparse_blocks=mb)
    assert np.array_equal(pi, permutation(g))
    assert blocks == plan(g).blocks
