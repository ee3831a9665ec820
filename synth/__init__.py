"""Seeded synthetic Q/K/V for the block-sparse video attention workloads.

This package only makes inputs. It holds none of the method's arithmetic: no
permutation, pooling, scoring, selection or attention. Both the CPU oracle
tests and the GPU path's tests and benchmark draw their inputs from here, so
the two sides always see the same bf16 bytes.
"""
from .workloads import WORKLOADS, Workload, get_workload
from .inputs import bf16_from_f32, bf16_to_f32, make_qkv, to_tnd, from_tnd

__all__ = ["WORKLOADS", "Workload", "get_workload", "bf16_from_f32", "bf16_to_f32",
           "make_qkv", "to_tnd", "from_tnd"]
