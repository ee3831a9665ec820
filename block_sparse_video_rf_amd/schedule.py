"""Which denoise steps and DiT layers take the sparse path.

"RainFusion Attention" (vLLM-Omni user guide), Configuration: ``start_step``
early denoise steps and ``end_step`` final denoise steps stay dense, and so do
the DiT blocks named by ``skip_layers`` (a selector such as ``"0-3,38"``);
everything else runs RainFusion. The introduction of the same page sends the
dense calls to full attention, which here is ``dense_attention`` (the
library's ``rf_dense_attn``). The same introduction sends calls without a
usable video geometry (no grid, fewer than 32 sparse blocks, sparsity 0) to
full attention too: ``rf_plan`` reports those as ``dense_fallback``, and
``scheduled_attention`` routes them to the dense path whatever the schedule.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import FrozenSet, Tuple


def parse_layers(selector) -> FrozenSet[int]:
    """Layer selector -> set of layer indices.

    Accepts ``None``/``""`` (no layer), a comma-separated string of indices and
    inclusive ranges (``"0-3,38"`` -> {0, 1, 2, 3, 38}), or an iterable of ints.
    Raises ValueError on negative indices, reversed ranges or malformed items.
    """
    if selector is None:
        return frozenset()
    if not isinstance(selector, str):
        out = set()
        for x in selector:
            if isinstance(x, bool) or not isinstance(x, int) or x < 0:
                raise ValueError(f"layer index must be a non-negative int, got {x!r}")
            out.add(x)
        return frozenset(out)
    out = set()
    for item in selector.replace(" ", "").split(","):
        if item == "":
            continue
        if "-" in item:
            lo, sep, hi = item.partition("-")
            if not (lo.isdigit() and hi.isdigit()):
                raise ValueError(f"bad layer range {item!r} in {selector!r}")
            a, b = int(lo), int(hi)
            if a > b:
                raise ValueError(f"reversed layer range {item!r} in {selector!r}")
            out.update(range(a, b + 1))
        else:
            if not item.isdigit():
                raise ValueError(f"bad layer index {item!r} in {selector!r}")
            out.add(int(item))
    return frozenset(out)


@dataclass(frozen=True)
class DenseSchedule:
    """``start_step``, ``end_step`` (integers >= 0) and ``skip_layers``."""

    start_step: int = 0
    end_step: int = 0
    skip_layers: FrozenSet[int] = field(default_factory=frozenset)

    def __post_init__(self):
        for name in ("start_step", "end_step"):
            val = getattr(self, name)
            if isinstance(val, bool) or not isinstance(val, int) or val < 0:
                raise ValueError(f"{name} must be an integer >= 0, got {val!r}")
        object.__setattr__(self, "skip_layers", parse_layers(self.skip_layers))

    def sparse(self, step: int, num_steps: int, layer: int) -> bool:
        """True if denoise step ``step`` (0-based, of ``num_steps``) at DiT
        block ``layer`` takes the sparse path."""
        if not (0 <= step < num_steps):
            raise ValueError(f"step {step} outside [0, {num_steps})")
        if layer < 0:
            raise ValueError(f"layer must be >= 0, got {layer}")
        if step < self.start_step or step >= num_steps - self.end_step:
            return False
        return layer not in self.skip_layers


def route(schedule: DenseSchedule, precision: str, step: int, num_steps: int,
          layer: int) -> Tuple[str, str]:
    """``("sparse" | "dense", precision)`` of one forward: the dense schedule
    decides the path; both paths run in the configured precision (the page
    shares it between the dense and sparse paths)."""
    if not schedule.sparse(step, num_steps, layer):
        return "dense", precision
    return "sparse", precision


def scheduled_attention(q, k, v, desc, schedule: DenseSchedule, step: int, num_steps: int,
                        layer: int, bufs=None, out=None, stream=None):
    """``attention`` on the steps and layers the schedule makes sparse,
    ``dense_attention`` on the others and on geometry fallbacks. Returns
    (out, bufs, sparse?); ``bufs`` serve both paths and are reused when they
    match the next call's descriptor."""
    from .rf import Buffers, attention, dense_attention
    path, _ = route(schedule, desc.precision, step, num_steps, layer)
    if bufs is None or bufs.desc != desc:  # buffers that serve both paths of this precision
        bufs = Buffers(desc, device=q.device, lists=True)
    if path == "sparse" and not bufs.info.dense_fallback:
        out, bufs = attention(q, k, v, desc, bufs=bufs, out=out, stream=stream)
        return out, bufs, True
    out, bufs = dense_attention(q, k, v, desc, bufs=bufs, out=out, stream=stream)
    return out, bufs, False
