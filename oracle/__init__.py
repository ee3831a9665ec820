"""CPU oracle for the RainFusion v2 block-sparse video attention path.

TEST INFRASTRUCTURE. This package is the plain, slow, obviously-correct
statement of what the path computes, used only to check the HIP path. Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. The product path (the HIP library and its Python
binding) never imports or calls it, and it imports nothing from them.

Precision: inputs are bf16 values; the oracle widens them to float64 and does
every step (pooling, scores, logits, softmax, PV) in float64. The e4m3 codec
works in exact float64 arithmetic from the OCP FP8 definition, and the mix-mode
scale and pre-quantisation multiply are done in float32 exactly as stated in
``fp8.py`` (that precision decides integer codes, so both sides use it).

Sources (cited by page title and section throughout):

* "RainFusion Attention" - the vLLM-Omni user-guide page for the
  ``RAINFUSION_ATTN`` backend: introduction, Configuration table, Requirements
  and compatibility, Geometry handling, Wan2.2 T2V quantization.
* "feat: add RainFusion sparse attention for wan2.2" - the xLLM pull request
  (commit summary; flag list).
* "aclnnRainFusionAttention" - the CANN operator reference: Formula and the
  constraint list.
* "RainFusion2.0: Temporal-Spatial Awareness and Hardware-Efficient
  Block-wise Sparse Attention" - the paper abstract.
* "MXAttention: Data-Free Optimal Scaling and Pre-Normalization Quantization
  for MXFP4 Attention" - the abstract (the 7.25 scaling boundary; quantising
  the exponentials before the row sum).

Parity pins: every function here is pinned by a CPU test in
``tests/test_oracle_*.py`` against page facts, closed forms, brute force or an
independent library routine. The one part with no pin is end-to-end video
quality (it needs trained models and a video benchmark): parity unpinned.
"""
from .geometry import Geometry, plan, permutation, permute_rows, unpermute_rows, block_rows
from .select import pool_blocks, block_scores, topk_sparse, select_lists, num_kept
from .attention import sparse_attention, attention_block, attention_block_fp8p, attention_block_mxp
from .fp8 import (e4m3_decode, e4m3_encode, e4m3_round, quantize_blocks, quantize_blocks_pow2,
                  pow2_scale_exponent)
from .mxfp4 import (e2m1_decode, e2m1_encode, e2m1_round, mx_scale_exponent, quantize_rows_mx,
                    quantize_v_mx, dequantize_rows_mx, dequantize_v_mx, mx_round_groups)
from .pipeline import run

__all__ = [
    "Geometry", "plan", "permutation", "permute_rows", "unpermute_rows", "block_rows",
    "pool_blocks", "block_scores", "topk_sparse", "select_lists", "num_kept",
    "sparse_attention", "attention_block", "attention_block_fp8p", "e4m3_decode",
    "e4m3_encode", "e4m3_round", "quantize_blocks", "quantize_blocks_pow2",
    "pow2_scale_exponent", "run", "attention_block_mxp", "e2m1_decode", "e2m1_encode",
    "e2m1_round", "mx_scale_exponent", "quantize_rows_mx", "quantize_v_mx", "dequantize_rows_mx",
    "dequantize_v_mx", "mx_round_groups",
]
