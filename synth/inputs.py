"""Seeded bf16 Q/K/V generator.

Recipe (the same for every consumer):

* Generator tree: ``SeedSequence(seed)`` spawns one child per tensor in the
  order Q, K, V. Each tensor's child spawns ``1 + B*N`` grandchildren: the
  first draws the smooth-component parameters, grandchild ``1 + b*N + n``
  draws the noise of batch item ``b``, head ``n``. The bytes therefore do not
  depend on how many threads fill them.
* Noise: standard normal, float32, one ``[S, D]`` slab per (batch, head),
  rows in natural order (prefix rows first, then video token (t, h, w) at
  ``prefix + (t*H + h)*W + w``, w fastest).
* Smooth component (only when the workload asks for it): for each head and
  channel d draw integer frequencies (ft, fh, fw) in {0, 1, 2} and a phase
  phi ~ U[0, 2*pi), then add ``0.5*cos(2*pi*(ft*t/T + fh*h/H + fw*w/W) + phi)``
  to every video row. Prefix rows get no component.
* Round once to bf16 (round to nearest, ties to even). The returned arrays
  hold bf16 bit patterns as ``uint16`` in BNSD layout ``[B, N, S, D]``.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .workloads import Workload


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def to_tnd(x: np.ndarray) -> np.ndarray:
    """BNSD ``[B, N, S, D]`` -> TND ``[B*S, N, D]`` (a copy)."""
    b, n, s, d = x.shape
    return np.ascontiguousarray(x.transpose(0, 2, 1, 3)).reshape(b * s, n, d)


def from_tnd(x: np.ndarray, batch: int) -> np.ndarray:
    """TND ``[B*S, N, D]`` -> BNSD ``[B, N, S, D]`` (a copy)."""
    t, n, d = x.shape
    return np.ascontiguousarray(x.reshape(batch, t // batch, n, d).transpose(0, 2, 1, 3))


def _smooth_component(grid, params):
    """``[T*H*W, D]`` float32 low-frequency field for one head."""
    T, H, W = grid
    ft, fh, fw, phi = params
    et = np.exp(2j * np.pi * np.outer(np.arange(T), ft) / T).astype(np.complex64)
    eh = np.exp(2j * np.pi * np.outer(np.arange(H), fh) / H).astype(np.complex64)
    ew = (np.exp(2j * np.pi * np.outer(np.arange(W), fw) / W) * np.exp(1j * phi)).astype(
        np.complex64)
    field = et[:, None, None, :] * eh[None, :, None, :] * ew[None, None, :, :]
    return (np.float32(0.5) * field.real).reshape(T * H * W, -1)


def _one_tensor(seq: np.random.SeedSequence, batch: int, heads: int, seq_len: int, dim: int,
                prefix: int, grid, smooth: bool, pool: ThreadPoolExecutor) -> np.ndarray:
    children = seq.spawn(1 + batch * heads)
    pg = np.random.default_rng(children[0])
    freqs = pg.integers(0, 3, size=(batch, heads, 3, dim))
    phases = pg.uniform(0.0, 2.0 * np.pi, size=(batch, heads, dim))
    out = np.empty((batch, heads, seq_len, dim), dtype=np.uint16)

    def fill(bn):
        b, n = divmod(bn, heads)
        x = np.random.default_rng(children[1 + bn]).standard_normal((seq_len, dim),
                                                                     dtype=np.float32)
        if smooth:
            f = freqs[b, n]
            x[prefix:] += _smooth_component(grid, (f[0], f[1], f[2], phases[b, n]))
        out[b, n] = bf16_from_f32(x)

    list(pool.map(fill, range(batch * heads)))
    return out


def make_qkv(w: Workload, seed: int | None = None, threads: int | None = None):
    """Return ``(q, k, v)`` as bf16 bit arrays in BNSD layout for workload ``w``."""
    seed = w.seed if seed is None else seed
    if threads is None:
        threads = max(1, min(16, os.cpu_count() or 1))
    sq, sk, sv = np.random.SeedSequence(seed).spawn(3)
    with ThreadPoolExecutor(max_workers=threads) as pool:
        args = (w.seq_len, w.head_dim, w.prefix_len, w.grid, w.smooth, pool)
        q = _one_tensor(sq, w.batch, w.heads_q, *args)
        k = _one_tensor(sk, w.batch, w.heads_kv, *args)
        v = _one_tensor(sv, w.batch, w.heads_kv, *args)
    return q, k, v
