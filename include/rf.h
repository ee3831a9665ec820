/*
 * rf.h - C ABI of the RainFusion v2 block-sparse video attention path for
 * AMD Instinct MI355X (gfx950).
 *
 * The path has five steps, each an entry point below except the host-only
 * plan:
 *   rf_plan         host: validate a call, derive the arrangement and sizes
 *   rf_permute      arrange Q/K/V into 128-token space-time blocks, pool the
 *                   sparse blocks, and (mix, fp8, mxfp4 precision) quantise
 *   rf_pool_select  score pooled blocks and build selectIdx / selectNum
 *   rf_sparse_attn  exact softmax attention restricted to the listed blocks
 *   rf_dense_attn   the same attention over every block (the dense path)
 *   rf_unpermute    undo the arrangement
 *
 * Sources (cited by page title and section):
 *   [RFA]  "RainFusion Attention" (vLLM-Omni user guide for the
 *          RAINFUSION_ATTN backend): introduction, Configuration, Geometry
 *          handling.
 *   [XPR]  "feat: add RainFusion sparse attention for wan2.2" (xLLM pull
 *          request): commit summary (frame-pairing rearrange, roundtrip).
 *   [ACL]  "aclnnRainFusionAttention" (CANN operator reference): Formula,
 *          the two-phase workspace/execute pattern, the constraint list.
 *   [RF2]  "RainFusion2.0: Temporal-Spatial Awareness and Hardware-Efficient
 *          Block-wise Sparse Attention": abstract (block-mean representative
 *          tokens, spatiotemporal permutation, first-frame sink).
 *   [MXA]  "MXAttention: Data-Free Optimal Scaling and Pre-Normalization
 *          Quantization for MXFP4 Attention" (catalyzex author page):
 *          abstract (softmax exponentials quantised before the row sum; the
 *          power-of-two scaling boundary 7.25 for MXFP4).
 *
 * Conventions for every entry point:
 *   - The caller owns all memory. Device pointers point to HIP device memory
 *     of the current device; the library never allocates, frees or
 *     synchronises. Its only mutable global state is the per-device address of
 *     rf_pool_select_noalloc's fixed array, set once under a lock (calls are
 *     thread-safe; see that entry point for what its shared array means).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is only enqueued on it.
 *   - Every argument is validated on the host before anything is enqueued;
 *     on any error nothing is enqueued and the status says why.
 *   - Launch failures return RF_ERR_HIP.
 *   - Results are deterministic: no floating-point atomics anywhere ([ACL]
 *     constraints: deterministic by default).
 *   - Outputs never alias inputs (out-of-place only).
 *
 * Element types: Q, K, V and the output are bf16 (raw 16-bit patterns);
 * [ACL] also allows fp16, which this library rejects (RF_ERR_DTYPE).
 */
#ifndef RF_H_
#define RF_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rf_status {
  RF_OK = 0,
  RF_ERR_NULL = 1,         /* a required pointer is NULL */
  RF_ERR_LAYOUT = 2,       /* layout is neither BNSD nor TND ([ACL] constraints) */
  RF_ERR_DTYPE = 3,        /* element type other than bf16 */
  RF_ERR_SHAPE = 4,        /* batch/heads/head_dim/seq_len out of range */
  RF_ERR_BLOCK_SHAPE = 5,  /* block shape not {128, 128} ([ACL]: entries > 0; only 128 built) */
  RF_ERR_GQA = 6,          /* heads_q not a multiple of heads_kv ([ACL] constraints) */
  RF_ERR_SPARSITY = 7,     /* sparsity not finite or outside [0, 1] ([RFA] Configuration) */
  RF_ERR_GEOMETRY = 8,     /* grid / prefix / first frame inconsistent with seq_len */
  RF_ERR_WORKSPACE = 9,    /* workspace smaller than rf_plan says */
  RF_ERR_UNSUPPORTED = 10, /* valid per the pages but not built here (see the field docs) */
  RF_ERR_PRECISION = 11,   /* unknown precision, or a buffer its precision needs is NULL */
  RF_ERR_HIP = 12,         /* a HIP launch failed */
  RF_ERR_ALIAS = 13,       /* an output aliases an input */
  RF_ERR_SCRATCH = 14      /* the call needs more scratch than rf_pool_select_noalloc's fixed
                              device array holds (RF_NOALLOC_SCRATCH_BYTES) */
} rf_status;

/* Size of the fixed device array that rf_pool_select_noalloc uses as its
 * workspace (72 MiB: the block scores of 8 heads x 1440 x 1440 sparse blocks
 * plus recomputed pools fit). */
#define RF_NOALLOC_SCRATCH_BYTES ((size_t)72 << 20)

typedef enum rf_layout {
  RF_LAYOUT_BNSD = 0, /* [B, N, S, D], rows of D contiguous */
  RF_LAYOUT_TND = 1   /* [B*S, N, D]: token-major, batch items stacked */
} rf_layout;

typedef enum rf_dtype { RF_DTYPE_BF16 = 0, RF_DTYPE_FP16 = 1 /* rejected */ } rf_dtype;

typedef enum rf_precision {
  RF_PREC_BF16 = 0, /* bf16 Q/K/V, bf16 MFMA, fp32 softmax ([ACL]: fp32 softmax for bf16) */
  RF_PREC_MIX = 1,  /* Q/K as fp8 E4M3 with one fp32 scale per (batch, head, 128-row
                       block); V, probabilities and output bf16; fp32 softmax.
                       [RFA] Configuration names "mix" without defining it. */
  RF_PREC_FP8 = 2,  /* all operands E4M3. [RFA] Configuration names "fp8" without defining it.
                       Q/K as in mix; V per (batch, kv head, 128-row block) with a
                       power-of-two scale 2^e, e the smallest integer with
                       amax <= 448 * 2^e (clamped to [-126, 127]; 0 for a zero block),
                       code = E4M3(x / 2^e); probabilities: each row's unnormalised
                       exponentials 2^t (t = scale*<q,k>/ln 2) quantised before the row
                       sum ([MXA]) with the same power-of-two block scale rule,
                       P = E4M3(2^(t - m)), m = ceil(row max of t - log2 448) (largest P
                       in (224, 448]), and out = sum P v / sum P (the sum of the rounded P).
                       Softmax bookkeeping and accumulation fp32, output bf16. */
  RF_PREC_MXFP4 = 3 /* all operands OCP MXFP4: E2M1 values in blocks of 32 along each
                       product's contraction, one E8M0 power-of-two scale 2^e per block.
                       [RFA] Wan2.2 T2V quantization names "mxfp4" for the sparse operator;
                       [MXA] gives the scale rule: e is the smallest integer with
                       amax <= 7.25 * 2^e (clamped to [-127, 127]; -127 for a zero block),
                       code = E2M1(x / 2^e), nearest-even, saturating at +-6. Blocks: 32
                       channels of each Q and K row; for V and P the four 32-key quarters
                       of each 128-row block (a short block's quarters hold its real rows).
                       P = MXFP4 of 2^(t - M) with t as in fp8 and M = ceil(row max of t)
                       (any integer M gives the same result), out = sum P v / sum P
                       ([MXA]). No rotation
                       ([RFA] mentions a default rotation policy without defining it).
                       Softmax bookkeeping and accumulation fp32, output bf16. */
} rf_precision;

/* One attention call. Sizes are per batch item; all batch items share the
 * same geometry. */
typedef struct rf_desc {
  int32_t layout;            /* rf_layout, for q/k/v and the final output */
  int32_t dtype;             /* rf_dtype; only RF_DTYPE_BF16 */
  int32_t batch;             /* B >= 1 */
  int32_t heads_q;           /* N1 >= 1 */
  int32_t heads_kv;          /* N2 >= 1, N1 % N2 == 0; query head n uses KV head n / (N1/N2) */
  int32_t head_dim;          /* D: 64 or 128 */
  int64_t seq_len;           /* S rows per batch item; S * head_dim * 2 < 2^31 */
  int32_t block_shape[2];    /* {blockShapeX, blockShapeY} ([ACL]); must be {128, 128} */
  int64_t prefix_len;        /* rows before the video (text, conditions, audio): always dense ([RFA]) */
  int64_t first_frame_rows;  /* 0, or grid_h*grid_w: first latent frame is the dense sink ([RF2]) */
  int32_t grid_t, grid_h, grid_w; /* latent video grid; all 0 = no geometry -> dense */
  int32_t precision;         /* rf_precision */
  double sparsity;           /* nominal dropped fraction of sparse key blocks, finite, in [0, 1] ([RFA]) */
  float scale;               /* softmax scale > 0 (usually 1/sqrt(D)) */
  int32_t min_sparse_blocks; /* fewer sparse blocks than this -> dense; [RFA] uses 32; <= 0 means 32 */
} rf_desc;

/* What rf_plan derives (all host-side). Block ids run over the permuted
 * sequence: head blocks [0, n_head), sparse blocks [n_head, n_head+n_sparse),
 * tail blocks after. */
typedef struct rf_plan_info {
  int32_t dense_fallback;   /* 1: every query block attends to every block ([RFA] introduction) */
  int32_t n_blocks;         /* n_head + n_sparse + n_tail */
  int32_t n_head;           /* ceil((prefix_len + first_frame_rows) / 128) */
  int32_t n_sparse;         /* frame pairs x (grid_h/8) x (grid_w/8) */
  int32_t n_tail;           /* ceil(promoted_rows / 128) */
  int32_t topk;             /* sparse key blocks kept per sparse query block:
                               n_sparse - floor(sparsity*n_sparse + 1e-6) */
  int32_t max_kv_blocks;    /* width of selectIdx: n_blocks */
  int32_t select_rows;      /* rows of selectIdx / selectNum: batch * n_blocks */
  int64_t head_rows;        /* prefix + first frame (seq_len on fallback) */
  int64_t sparse_rows;      /* 128 * n_sparse */
  int64_t promoted_rows;    /* video rows moved to the dense tail ([RFA] Geometry handling) */
  int64_t qp_elems;         /* bf16 elements of qp / out_p: batch*heads_q*seq_len*head_dim */
  int64_t kp_elems;         /* bf16 elements of kp: batch*heads_kv*seq_len*head_dim */
  int64_t vpt_elems;        /* elements of vpt: batch*heads_kv*n_blocks*head_dim*128
                               (bf16; one-byte E4M3 codes in fp8 precision) */
  int64_t q_pool_elems;     /* fp32 elements of q_pool: batch*heads_q*n_sparse*head_dim */
  int64_t k_pool_elems;     /* fp32 elements of k_pool: batch*heads_kv*n_sparse*head_dim */
  int64_t q_scale_elems;    /* fp32 elements of q_scale (mix): batch*heads_q*n_blocks */
  int64_t k_scale_elems;    /* fp32 elements of k_scale (mix): batch*heads_kv*n_blocks */
  int64_t v_scale_elems;    /* fp32 elements of v_scale (fp8): batch*heads_kv*n_blocks */
  size_t ws_select_bytes;   /* workspace of rf_pool_select */
  /* Bytes of the precision-dependent buffers for desc->precision (0 where the
   * precision does not use the buffer). Every size is the buffer's natural
   * size: the attention kernel reads nothing past the real rows of any buffer
   * (a K tile that runs past the end of the sequence reads zeros instead).
   *           bf16        mix            fp8            mxfp4
   *   q8      0           qp_elems       qp_elems       qp_elems / 2
   *   k8      0           kp_elems       kp_elems       kp_elems / 2
   *   vpt     2*vpt_elems 2*vpt_elems    vpt_elems      vpt_elems / 2
   *   q_scale 0           4*q_scale_elems 4*q_scale_elems qp_elems / 32
   *   k_scale 0           4*k_scale_elems 4*k_scale_elems kp_elems / 32
   *   v_scale 0           0              4*v_scale_elems batch*heads_kv*n_blocks*4*head_dim */
  int64_t q8_bytes, k8_bytes, vpt_bytes, q_scale_bytes, k_scale_bytes, v_scale_bytes;
  int64_t kp_bytes;         /* bytes of kp: 2 * kp_elems */
} rf_plan_info;

/* Validate `desc` and derive the arrangement. Host only: touches no device,
 * so it can run on a machine without a GPU. */
rf_status rf_plan(const rf_desc* desc, rf_plan_info* info);

/* Step 1 (+ pooling, + quantisation). [RFA] introduction and Geometry
 * handling; [XPR] commit summary (frame pairs, one call for Q, K and V);
 * [RF2] abstract (spatiotemporal permutation, block means).
 *
 * Permuted order of each batch item: prefix rows; the first frame (if any);
 * the sparse blocks, each one 2 frames x 8x8 tile box numbered (pair, tile
 * row, tile column), tokens (dt, dh, dw) in raster order; then the promoted
 * rows (those that fit no box) in natural order. Video token (t, h, w) sits
 * at natural row prefix_len + (t*grid_h + h)*grid_w + w.
 *
 * Inputs (device, caller layout): q [.., heads_q, ..], k and v [.., heads_kv, ..].
 * Any of q, k, v may be NULL to skip that tensor.
 * Outputs (device), all optional unless stated:
 *   qp     bf16 [B, N1, S, D] permuted rows (BNSD whatever the input layout)
 *   kp     bf16 [B, N2, S, D]
 *   vpt    bf16 [B, N2, n_blocks, D, 128]: V block-transposed, vpt[b,n,j,d,c]
 *          = V row c of block j, channel d; columns c >= the block's length are 0.
 *          Required when v is given (it is the layout rf_sparse_attn reads).
 *   q_pool fp32 [B, N1, n_sparse, D] mean of each sparse block of Q
 *   k_pool fp32 [B, N2, n_sparse, D] mean of each sparse block of K
 *   q8,k8  uint8 E4M3 codes, same shape as qp/kp   (mix, fp8; required there)
 *   q_scale,k_scale fp32 [B, N, n_blocks] per-block scales (mix, fp8; required)
 *   v_scale fp32 [B, N2, n_blocks] power-of-two V scales (fp8; required when v
 *          is given; ignored otherwise). In fp8 precision vpt holds one-byte
 *          E4M3 codes of V / v_scale in the same block-transposed layout.
 * mxfp4 (RF_PREC_MXFP4; every buffer below required for a given input):
 *   q8,k8   E2M1 codes, two per byte (channel 2i in the low nibble):
 *           [B, N, S, D/2] bytes
 *   q_scale,k_scale E8M0 exponents (e + 127) of each row's 32-channel blocks:
 *           [B, N, S, D/32] bytes
 *   vpt     E2M1 codes of V^T, two keys per byte (key 2i in the low nibble):
 *           [B, N2, n_blocks, D, 64] bytes; keys past the block's end are 0
 *   v_scale E8M0 exponents of V's key quarters: [B, N2, n_blocks, 4, D] bytes,
 *           channel d = 32 a + i of quarter g at position (D/32) i + a of row
 *           g (the order in which the attention kernel reads them)
 * Sizes of every buffer: rf_plan_info (q8_bytes .. v_scale_bytes).
 * Mix quantisation of a block: amax = max |x|; r = 448.0f / amax;
 * code = E4M3 round-to-nearest-even, saturating at 448, of (float)(x * r);
 * scale = amax / 448.0f; an all-zero block gets r = scale = 1.
 * Errors: RF_ERR_NULL (a given input has no output), RF_ERR_PRECISION (a
 * buffer the precision needs is NULL), RF_ERR_ALIAS (an output overlaps an
 * input), plus the descriptor errors of rf_plan. */
rf_status rf_permute(const rf_desc* desc, const void* q, const void* k, const void* v,
                     void* qp, void* kp, void* vpt, float* q_pool, float* k_pool,
                     uint8_t* q8, uint8_t* k8, void* q_scale, void* k_scale, void* v_scale,
                     void* stream);

/* Steps 2-3. [RFA] introduction (pool 128-token blocks, rank per query
 * block, keep the highest-scoring); [RF2] abstract (block means as
 * representative tokens); [ACL] constraints (selectIdx [T, heads, maxKv]
 * with T = batch * query blocks, -1 fill; selectNum [T, heads]).
 *
 * q_pool / k_pool: pooled blocks as written by rf_permute. If either is NULL
 * it is recomputed from qp / kp into the workspace.
 * Score of query block i against key block j, query head n:
 *   scale * <q_pool[n, i], k_pool[n / G, j]>  (fp32).
 * A sparse query block keeps the topk highest-scoring sparse key blocks
 * (equal scores: lower id first) plus every head and tail block; its list is
 * sorted ascending. Head and tail query blocks list every block. Unused list
 * entries are -1.
 * Outputs: select_idx int32 [select_rows, N1, max_kv] (max_kv >= n_blocks),
 *          select_num int32 [select_rows, N1].
 * Workspace: device, at least ws_select_bytes (from rf_plan). */
rf_status rf_pool_select(const rf_desc* desc, const void* qp, const void* kp,
                         const float* q_pool, const float* k_pool, int32_t* select_idx,
                         int32_t* select_num, int32_t max_kv, void* workspace,
                         size_t workspace_bytes, void* stream);

/* rf_pool_select for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, outputs and errors as rf_pool_select, without the workspace: the
 * block scores (and pooled blocks, when q_pool or k_pool is NULL) go to a fixed
 * device array inside the library of RF_NOALLOC_SCRATCH_BYTES, one per device,
 * which each device holds from the first call on it until the process ends.
 * The call allocates and frees nothing (no hipMalloc, hipFree or allocating
 * library routine); its first call on a device only looks up that device's
 * array address (hipGetSymbolAddress, with that device current).
 * Space needed: the scores, B*N1*n_sparse^2 floats, plus B*N1*n_sparse*D
 * floats if q_pool is NULL, plus (B*N1 + B*N2)*n_sparse*D floats if k_pool is
 * NULL (each piece rounded up to 256 bytes); more than the array holds returns
 * RF_ERR_SCRATCH before anything is enqueued. Every piece is written before it
 * is read, so nothing carries over from an earlier call.
 * All calls on one device share its array: calls whose work can overlap on
 * that device (other streams, other host threads) race on it; the caller must
 * order them (for instance, one stream). */
rf_status rf_pool_select_noalloc(const rf_desc* desc, const void* qp, const void* kp,
                                 const float* q_pool, const float* k_pool, int32_t* select_idx,
                                 int32_t* select_num, int32_t max_kv, void* stream);

/* Step 4. [ACL] Formula: out = softmax(scale * Q K^T) V over the key rows of
 * the listed 128x128 blocks (no additive mask; short blocks contribute only
 * their real rows). fp32 accumulation and fp32 online softmax.
 * bf16 precision reads qp, kp, vpt; mix precision reads q8, k8, q_scale,
 * k_scale, vpt (logits = scale * q_scale * k_scale * <q8, k8>); fp8 precision
 * also reads v_scale, with vpt as E4M3 codes, and quantises P (see
 * RF_PREC_FP8); mxfp4 reads q8, k8, q_scale, k_scale, vpt and v_scale in the
 * layouts rf_permute writes for it and quantises P (see RF_PREC_MXFP4).
 * Scale arguments are fp32 arrays (mix, fp8) or E8M0 byte arrays (mxfp4).
 * Arguments a precision does not read may be NULL.
 * select_idx / select_num as above (any list the caller builds is accepted:
 * entries outside [0, n_blocks) contribute nothing, exactly as if skipped,
 * provided V holds finite values; counts are clamped to max_kv).
 * A row with an empty list gets zeros.
 * out_p: bf16 [B, N1, S, D], permuted row order, rounded to nearest even. */
rf_status rf_sparse_attn(const rf_desc* desc, const void* qp, const void* kp, const void* vpt,
                         const uint8_t* q8, const uint8_t* k8, const void* q_scale,
                         const void* k_scale, const void* v_scale, const int32_t* select_idx,
                         const int32_t* select_num, int32_t max_kv, void* out_p, void* stream);

/* Dense path. [RFA] introduction: calls that RainFusion does not handle, and
 * the steps and layers its Configuration keeps dense (start_step, end_step,
 * skip_layers), delegate to full attention (FLASH_ATTN there).
 * out = softmax(scale * Q K^T) V over every key row of the sequence, computed
 * on the same buffers as rf_sparse_attn with every block listed in order. No
 * list is read, so none needs to be built. Full attention does not depend on
 * the order of the keys, so any arrangement that rf_permute made gives the
 * same result (after rf_unpermute) as full attention in the caller's order.
 * Arguments, layouts and errors as rf_sparse_attn without the lists.
 * out_p: bf16 [B, N1, S, D], permuted row order, rounded to nearest even. */
rf_status rf_dense_attn(const rf_desc* desc, const void* qp, const void* kp, const void* vpt,
                        const uint8_t* q8, const uint8_t* k8, const void* q_scale,
                        const void* k_scale, const void* v_scale, void* out_p, void* stream);

/* Step 5. [XPR] commit summary (inverse rearrange; roundtrip check).
 * out[natural row pi(r)] = out_p[r]; out in the caller's layout with heads_q
 * heads. */
rf_status rf_unpermute(const rf_desc* desc, const void* out_p, void* out, void* stream);

/* Short English text for a status code (static storage). */
const char* rf_status_str(rf_status status);

/* Library version string (static storage). */
const char* rf_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RF_H_ */
