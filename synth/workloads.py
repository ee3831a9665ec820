"""The five synthetic workloads, named by what they are.

Shapes follow the video DiT workloads that the RainFusion pages speak of
(vLLM-Omni "RainFusion Attention" page: MiniMax-H3 at 1344x768 gives the
latent grid (62, 24, 42); Wan2.2 text-to-video at 720p gives (21, 40, 64)).
No model weights or activations are used: values are seeded noise plus, for
the large shapes, a smooth low-frequency component over (t, h, w) so that
block means carry information (see ``inputs.py``).

``first_frame`` says whether the first latent frame is split off as the
always-dense sink; ``smooth`` whether the low-frequency component is added.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    prefix_len: int
    grid: Tuple[int, int, int]
    first_frame: bool
    sparsity: float
    precision: str  # "bf16" or "mix"
    smooth: bool
    seed: int

    @property
    def video_len(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def seq_len(self) -> int:
        return self.prefix_len + self.video_len

    @property
    def first_frame_rows(self) -> int:
        return self.grid[1] * self.grid[2] if self.first_frame else 0

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # 2 heads, D=64, 128-row prefix + grid (9,16,32); pure N(0,1).
    "tiny": Workload("tiny", 1, 2, 2, 64, 128, (9, 16, 32), True, 0.8, "bf16", False, 1001),
    # Wan2.2-style 8x8-aligned latent grid, 40 heads, D=128.
    "wan22": Workload("wan22", 1, 40, 40, 128, 512, (21, 40, 64), True, 0.8, "bf16", True, 1002),
    # MiniMax-H3 at 1344x768: w=42 is not a multiple of 8, so a suffix is promoted.
    "minimax_h3": Workload("minimax_h3", 1, 24, 24, 128, 512, (62, 24, 42), False, 0.8, "bf16",
                           True, 1003),
    # The Wan2.2 shapes and data, with fp8 e4m3 Q/K ("mix" precision).
    "wan22_mix": Workload("wan22_mix", 1, 40, 40, 128, 512, (21, 40, 64), True, 0.8, "mix", True,
                          1002),
    # The Wan2.2 shapes and data with every attention operand in fp8 e4m3 ("fp8").
    "wan22_fp8": Workload("wan22_fp8", 1, 40, 40, 128, 512, (21, 40, 64), True, 0.8, "fp8", True,
                          1002),
    # The Wan2.2 shapes and data with every attention operand in MXFP4 ("mxfp4").
    "wan22_mxfp4": Workload("wan22_mxfp4", 1, 40, 40, 128, 512, (21, 40, 64), True, 0.8, "mxfp4",
                            True, 1002),
    # Long video with grouped-query attention: 8 query heads share 2 KV heads.
    "gqa_long": Workload("gqa_long", 1, 8, 2, 128, 512, (31, 64, 96), True, 0.9, "bf16", True, 1005),
}


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None
