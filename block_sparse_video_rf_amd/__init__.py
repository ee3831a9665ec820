"""RainFusion v2 block-sparse video attention for AMD MI355X (gfx950).

The compute lives in the HIP library ``librf.so`` (C ABI in ``include/rf.h``);
``rf`` is its ctypes binding. PyTorch supplies device memory and streams only.
"""
from .rf import (Buffers, Desc, RfError, RfPlanInfo, attention, dense_attention, load_library,
                 rf_dense_attn, rf_permute, rf_plan, rf_pool_select, rf_pool_select_noalloc,
                 rf_sparse_attn, NOALLOC_SCRATCH_BYTES,
                 rf_status_str, rf_unpermute, rf_version, EXPORTS, LIB_PATH)
from .schedule import DenseSchedule, parse_layers, route, scheduled_attention

__all__ = ["Buffers", "DenseSchedule", "route", "Desc", "RfError", "RfPlanInfo", "attention",
           "dense_attention", "load_library", "parse_layers", "rf_dense_attn", "rf_permute",
           "rf_plan", "rf_pool_select", "rf_pool_select_noalloc", "rf_sparse_attn",
           "NOALLOC_SCRATCH_BYTES", "rf_status_str", "rf_unpermute",
           "rf_version", "scheduled_attention", "EXPORTS", "LIB_PATH"]
