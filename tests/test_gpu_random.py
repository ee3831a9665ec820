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


@pytest.mark.parametrize("seed", range(10))
def test_random_geometry(seed):
    w, extra = _case(seed)
    log(f"[random {seed}] {w}")
    full_check(w, extra)
