"""ctypes binding of ``librf.so`` (include/rf.h), same names as the C ABI.

Argument marshalling only: every step runs in the HIP library. PyTorch
tensors are used for device memory and the current HIP stream; their data
pointers go straight to the C entry points. There is no fallback of any
kind: if the library is missing or a call fails, a ``RuntimeError`` is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "librf.so")

LAYOUT_BNSD, LAYOUT_TND = 0, 1
DTYPE_BF16, DTYPE_FP16 = 0, 1
PREC_BF16, PREC_MIX, PREC_FP8, PREC_MXFP4 = 0, 1, 2, 3
_PREC = {"bf16": PREC_BF16, "mix": PREC_MIX, "fp8": PREC_FP8, "mxfp4": PREC_MXFP4}
_LAYOUT = {"BNSD": LAYOUT_BNSD, "TND": LAYOUT_TND}


class RfDesc(ctypes.Structure):
    _fields_ = [
        ("layout", ctypes.c_int32), ("dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("seq_len", ctypes.c_int64), ("block_shape", ctypes.c_int32 * 2),
        ("prefix_len", ctypes.c_int64), ("first_frame_rows", ctypes.c_int64),
        ("grid_t", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
        ("precision", ctypes.c_int32), ("sparsity", ctypes.c_double), ("scale", ctypes.c_float),
        ("min_sparse_blocks", ctypes.c_int32),
    ]


class RfPlanInfo(ctypes.Structure):
    _fields_ = [
        ("dense_fallback", ctypes.c_int32), ("n_blocks", ctypes.c_int32),
        ("n_head", ctypes.c_int32), ("n_sparse", ctypes.c_int32), ("n_tail", ctypes.c_int32),
        ("topk", ctypes.c_int32), ("max_kv_blocks", ctypes.c_int32),
        ("select_rows", ctypes.c_int32), ("head_rows", ctypes.c_int64),
        ("sparse_rows", ctypes.c_int64), ("promoted_rows", ctypes.c_int64),
        ("qp_elems", ctypes.c_int64), ("kp_elems", ctypes.c_int64), ("vpt_elems", ctypes.c_int64),
        ("q_pool_elems", ctypes.c_int64), ("k_pool_elems", ctypes.c_int64),
        ("q_scale_elems", ctypes.c_int64), ("k_scale_elems", ctypes.c_int64),
        ("v_scale_elems", ctypes.c_int64), ("ws_select_bytes", ctypes.c_size_t),
        ("q8_bytes", ctypes.c_int64), ("k8_bytes", ctypes.c_int64), ("vpt_bytes", ctypes.c_int64),
        ("q_scale_bytes", ctypes.c_int64), ("k_scale_bytes", ctypes.c_int64),
        ("v_scale_bytes", ctypes.c_int64), ("kp_bytes", ctypes.c_int64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


EXPORTS = ("rf_plan", "rf_permute", "rf_pool_select", "rf_pool_select_noalloc",
           "rf_sparse_attn", "rf_dense_attn", "rf_unpermute", "rf_status_str", "rf_version")

# Size of the fixed device array behind rf_pool_select_noalloc (RF_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 72 << 20

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load ``librf.so`` (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(run python -m block_sparse_video_rf_amd.build)")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    D = ctypes.POINTER(RfDesc)
    lib.rf_plan.argtypes = [D, ctypes.POINTER(RfPlanInfo)]
    lib.rf_permute.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.rf_pool_select.argtypes = [D, P, P, P, P, P, P, ctypes.c_int32, P, ctypes.c_size_t, P]
    lib.rf_pool_select_noalloc.argtypes = [D, P, P, P, P, P, P, ctypes.c_int32, P]
    lib.rf_sparse_attn.argtypes = [D, P, P, P, P, P, P, P, P, P, P, ctypes.c_int32, P, P]
    lib.rf_dense_attn.argtypes = [D, P, P, P, P, P, P, P, P, P, P]
    lib.rf_unpermute.argtypes = [D, P, P, P]
    for f in ("rf_plan", "rf_permute", "rf_pool_select", "rf_pool_select_noalloc",
              "rf_sparse_attn", "rf_dense_attn", "rf_unpermute"):
        getattr(lib, f).restype = ctypes.c_int
    lib.rf_status_str.argtypes = [ctypes.c_int]
    lib.rf_status_str.restype = ctypes.c_char_p
    lib.rf_version.argtypes = []
    lib.rf_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def rf_status_str(status: int) -> str:
    return load_library().rf_status_str(status).decode()


def rf_version() -> str:
    return load_library().rf_version().decode()


class RfError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {rf_status_str(status)} (status {status})")


def _check(fn: str, status: int):
    if status != 0:
        raise RfError(fn, status)


@dataclass
class Desc:
    """Python mirror of ``rf_desc``."""
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    seq_len: int
    prefix_len: int = 0
    first_frame_rows: int = 0
    grid: Tuple[int, int, int] = (0, 0, 0)
    sparsity: float = 0.8
    scale: Optional[float] = None
    precision: str = "bf16"
    layout: str = "BNSD"
    block_shape: Tuple[int, int] = (128, 128)
    min_sparse_blocks: int = 32
    dtype: int = DTYPE_BF16

    @classmethod
    def from_workload(cls, w, layout: str = "BNSD", **kw) -> "Desc":
        args = dict(batch=w.batch, heads_q=w.heads_q, heads_kv=w.heads_kv, head_dim=w.head_dim,
                    seq_len=w.seq_len, prefix_len=w.prefix_len,
                    first_frame_rows=w.first_frame_rows, grid=tuple(w.grid),
                    sparsity=w.sparsity, precision=w.precision, layout=layout)
        args.update(kw)
        return cls(**args)

    def c(self) -> RfDesc:
        d = RfDesc()
        d.layout = _LAYOUT[self.layout] if isinstance(self.layout, str) else int(self.layout)
        d.dtype = int(self.dtype)
        d.batch, d.heads_q, d.heads_kv = self.batch, self.heads_q, self.heads_kv
        d.head_dim, d.seq_len = self.head_dim, self.seq_len
        d.block_shape[0], d.block_shape[1] = self.block_shape
        d.prefix_len, d.first_frame_rows = self.prefix_len, self.first_frame_rows
        d.grid_t, d.grid_h, d.grid_w = self.grid
        d.precision = _PREC[self.precision] if isinstance(self.precision, str) else int(
            self.precision)
        d.sparsity = float(self.sparsity)
        d.scale = float(self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim))
        d.min_sparse_blocks = self.min_sparse_blocks
        return d


def rf_plan(desc: Desc) -> RfPlanInfo:
    info = RfPlanInfo()
    d = desc.c()
    _check("rf_plan", load_library().rf_plan(ctypes.byref(d), ctypes.byref(info)))
    return info


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def rf_permute(desc: Desc, q, k, v, qp=None, kp=None, vpt=None, q_pool=None, k_pool=None,
               q8=None, k8=None, q_scale=None, k_scale=None, v_scale=None, stream=None):
    d = desc.c()
    _check("rf_permute", load_library().rf_permute(
        ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(qp), _ptr(kp), _ptr(vpt), _ptr(q_pool),
        _ptr(k_pool), _ptr(q8), _ptr(k8), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
        _stream(stream)))


def rf_pool_select(desc: Desc, qp, kp, q_pool, k_pool, select_idx, select_num, max_kv: int,
                   workspace, workspace_bytes: Optional[int] = None, stream=None):
    d = desc.c()
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("rf_pool_select", load_library().rf_pool_select(
        ctypes.byref(d), _ptr(qp), _ptr(kp), _ptr(q_pool), _ptr(k_pool), _ptr(select_idx),
        _ptr(select_num), int(max_kv), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def rf_pool_select_noalloc(desc: Desc, qp, kp, q_pool, k_pool, select_idx, select_num,
                           max_kv: int, stream=None):
    """``rf_pool_select`` with the library's fixed device array as its workspace
    (no allocation anywhere; calls on one device share the array)."""
    d = desc.c()
    _check("rf_pool_select_noalloc", load_library().rf_pool_select_noalloc(
        ctypes.byref(d), _ptr(qp), _ptr(kp), _ptr(q_pool), _ptr(k_pool), _ptr(select_idx),
        _ptr(select_num), int(max_kv), _stream(stream)))


def rf_sparse_attn(desc: Desc, qp, kp, vpt, q8, k8, q_scale, k_scale, v_scale, select_idx,
                   select_num, max_kv: int, out_p, stream=None):
    d = desc.c()
    _check("rf_sparse_attn", load_library().rf_sparse_attn(
        ctypes.byref(d), _ptr(qp), _ptr(kp), _ptr(vpt), _ptr(q8), _ptr(k8), _ptr(q_scale),
        _ptr(k_scale), _ptr(v_scale), _ptr(select_idx), _ptr(select_num), int(max_kv),
        _ptr(out_p), _stream(stream)))


def rf_dense_attn(desc: Desc, qp, kp, vpt, q8, k8, q_scale, k_scale, v_scale, out_p,
                  stream=None):
    d = desc.c()
    _check("rf_dense_attn", load_library().rf_dense_attn(
        ctypes.byref(d), _ptr(qp), _ptr(kp), _ptr(vpt), _ptr(q8), _ptr(k8), _ptr(q_scale),
        _ptr(k_scale), _ptr(v_scale), _ptr(out_p), _stream(stream)))


def rf_unpermute(desc: Desc, out_p, out, stream=None):
    d = desc.c()
    _check("rf_unpermute", load_library().rf_unpermute(ctypes.byref(d), _ptr(out_p), _ptr(out),
                                                        _stream(stream)))


class Buffers:
    """Device buffers for one call shape, sized from ``rf_plan`` (torch allocations).

    ``lists=False`` leaves out what only the sparse path uses (pooled blocks,
    selectIdx / selectNum, the selection workspace): the dense path needs none.
    In mix and fp8 precision Q/K exist only as E4M3 codes (``q8``, ``k8``) with
    per-block scales; in fp8 ``vpt`` holds one-byte E4M3 codes and ``v_scale``
    their power-of-two block scales. In mxfp4 precision ``q8``, ``k8`` and
    ``vpt`` hold E2M1 codes two per byte and the scales are E8M0 bytes (one per
    32 channels of a Q/K row, one per channel and 32-key quarter of a V block).
    """

    def __init__(self, desc: Desc, device="cuda", lists: bool = True):
        import torch
        self.desc = desc
        self.info = info = rf_plan(desc)
        B, N1, N2, S, D = desc.batch, desc.heads_q, desc.heads_kv, desc.seq_len, desc.head_dim
        nB, nS = info.n_blocks, info.n_sparse
        bf = torch.bfloat16
        prec = _PREC[desc.precision] if isinstance(desc.precision, str) else int(desc.precision)
        mix = prec != PREC_BF16               # quantised Q/K
        v8 = prec in (PREC_FP8, PREC_MXFP4)   # quantised V
        f4 = prec == PREC_MXFP4
        u8, f32 = torch.uint8, torch.float32

        self.qp = None if mix else torch.empty((B, N1, S, D), dtype=bf, device=device)
        self.kp = None if mix else torch.empty((B, N2, S, D), dtype=bf, device=device)
        if f4:
            self.vpt = torch.empty((B, N2, nB, D, 64), dtype=u8, device=device)
            self.v_scale = torch.empty((B, N2, nB, 4, D), dtype=u8, device=device)
            self.q8 = torch.empty((B, N1, S, D // 2), dtype=u8, device=device)
            self.k8 = torch.empty((B, N2, S, D // 2), dtype=u8, device=device)
            self.q_scale = torch.empty((B, N1, S, D // 32), dtype=u8, device=device)
            self.k_scale = torch.empty((B, N2, S, D // 32), dtype=u8, device=device)
        else:
            self.vpt = torch.empty((B, N2, nB, D, 128), dtype=u8 if v8 else bf, device=device)
            self.v_scale = torch.empty((B, N2, nB), dtype=f32, device=device) if v8 else None
            self.q8 = torch.empty((B, N1, S, D), dtype=u8, device=device) if mix else None
            self.k8 = torch.empty((B, N2, S, D), dtype=u8, device=device) if mix else None
            self.q_scale = torch.empty((B, N1, nB), dtype=f32, device=device) if mix else None
            self.k_scale = torch.empty((B, N2, nB), dtype=f32, device=device) if mix else None
        # Every precision-dependent buffer has the size rf_plan gives for it.
        for name in ("q8", "k8", "vpt", "q_scale", "k_scale", "v_scale") + (() if mix else ("kp",)):
            t = getattr(self, name)
            nbytes = 0 if t is None else t.untyped_storage().nbytes()
            if nbytes != getattr(info, name + "_bytes"):
                raise AssertionError(f"{name}: {nbytes} bytes, rf_plan says {getattr(info, name + '_bytes')}")
        self.q_pool = torch.empty((B, N1, nS, D), dtype=f32, device=device) if lists else None
        self.k_pool = torch.empty((B, N2, nS, D), dtype=f32, device=device) if lists else None
        self.select_idx = (torch.empty((B * nB, N1, nB), dtype=torch.int32, device=device)
                           if lists else None)
        self.select_num = (torch.empty((B * nB, N1), dtype=torch.int32, device=device)
                           if lists else None)
        self.workspace = (torch.empty((max(1, info.ws_select_bytes),), dtype=torch.uint8,
                                      device=device) if lists else None)
        self.out_p = torch.empty((B, N1, S, D), dtype=bf, device=device)


def attention(q, k, v, desc: Desc, bufs: Optional[Buffers] = None, out=None, stream=None):
    """The whole path: permute -> pool/select -> sparse attention -> unpermute.

    ``q``, ``k``, ``v``: bf16 CUDA tensors in ``desc.layout``. Returns the
    output in the same layout (bf16) and the buffers used.
    """
    import torch
    if bufs is None:
        bufs = Buffers(desc, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    b = bufs
    rf_permute(desc, q, k, v, b.qp, b.kp, b.vpt, b.q_pool, b.k_pool, b.q8, b.k8, b.q_scale,
               b.k_scale, b.v_scale, stream=stream)
    nB = b.info.n_blocks
    rf_pool_select(desc, b.qp, b.kp, b.q_pool, b.k_pool, b.select_idx, b.select_num, nB,
                   b.workspace, stream=stream)
    rf_sparse_attn(desc, b.qp, b.kp, b.vpt, b.q8, b.k8, b.q_scale, b.k_scale, b.v_scale,
                   b.select_idx, b.select_num, nB, b.out_p, stream=stream)
    rf_unpermute(desc, b.out_p, out, stream=stream)
    return out, bufs


def dense_attention(q, k, v, desc: Desc, bufs: Optional[Buffers] = None, out=None, stream=None):
    """The dense path: permute -> attention over every block -> unpermute.

    Same inputs and output as ``attention``; no pooling, no selection, no
    lists. Full attention is independent of the key order, so the result is
    full attention in the caller's order (for mix and fp8 precision: with the
    same per-block E4M3 operands as the sparse path).
    """
    import torch
    if bufs is None:
        bufs = Buffers(desc, device=q.device, lists=False)
    if out is None:
        out = torch.empty_like(q)
    b = bufs
    rf_permute(desc, q, k, v, b.qp, b.kp, b.vpt, None, None, b.q8, b.k8, b.q_scale, b.k_scale,
               b.v_scale, stream=stream)
    rf_dense_attn(desc, b.qp, b.kp, b.vpt, b.q8, b.k8, b.q_scale, b.k_scale, b.v_scale,
                  b.out_p, stream=stream)
    rf_unpermute(desc, b.out_p, out, stream=stream)
    return out, bufs
