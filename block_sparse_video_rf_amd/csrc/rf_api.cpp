// Host side of the C ABI: validation, the arrangement plan, and argument
// checks before any launch. No HIP calls here; every entry point validates
// first and only then hands a derived RfGeom to the launchers.
//
// Plan rules ("RainFusion Attention" page: introduction, Configuration,
// Geometry handling; "aclnnRainFusionAttention": constraint list):
//   - the video is sparse only if it has a grid, sparsity > 0 and at least
//     min_sparse_blocks (32) full 2x8x8 blocks; otherwise the call is a plain
//     dense attention over the natural order;
//   - the first frame (if first_frame_rows = H*W) and the prefix are dense;
//   - rows that fit no box are promoted to a dense tail; nothing is padded;
//   - head and tail segments are cut into 128-row blocks by ceiling division;
//   - kept sparse blocks per sparse query block: n_sparse - floor(s*n_sparse + 1e-6).
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "rf_internal.h"

namespace {

bool valid_layout(int32_t l) { return l == RF_LAYOUT_BNSD || l == RF_LAYOUT_TND; }

// Switch for the mxfp4 kernels: when false the device entry points refuse the
// precision with RF_ERR_UNSUPPORTED (rf_plan still reports its buffer sizes).
constexpr bool kMxfp4Enabled = true;
bool mxfp4_off(const rf_desc* d) { return d->precision == RF_PREC_MXFP4 && !kMxfp4Enabled; }

// [a, a+na) and [b, b+nb) overlap (both non-empty, both non-null).
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

}  // namespace

rf_status rf_derive(const rf_desc* d, RfGeom* g, rf_plan_info* info) {
  if (!d) return RF_ERR_NULL;
  if (!valid_layout(d->layout)) return RF_ERR_LAYOUT;
  if (d->dtype != RF_DTYPE_BF16) return RF_ERR_DTYPE;
  if (d->batch < 1 || d->heads_q < 1 || d->heads_kv < 1 || d->seq_len < 1) return RF_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return RF_ERR_UNSUPPORTED;
  if (d->block_shape[0] <= 0 || d->block_shape[1] <= 0) return RF_ERR_BLOCK_SHAPE;
  if (d->block_shape[0] != 128 || d->block_shape[1] != 128) return RF_ERR_UNSUPPORTED;
  if (d->heads_q % d->heads_kv != 0) return RF_ERR_GQA;
  if (!isfinite(d->sparsity) || d->sparsity < 0.0 || d->sparsity > 1.0) return RF_ERR_SPARSITY;
  if (!isfinite(d->scale) || !(d->scale > 0.0f)) return RF_ERR_SHAPE;
  if (d->precision != RF_PREC_BF16 && d->precision != RF_PREC_MIX && d->precision != RF_PREC_FP8 &&
      d->precision != RF_PREC_MXFP4)
    return RF_ERR_PRECISION;
  // Per-(batch, head) row offsets are formed in 64-bit; keep counts in 32-bit ranges.
  if (d->seq_len > ((int64_t)1 << 31) - 128) return RF_ERR_SHAPE;
  // The attention kernel addresses one (batch, kv head)'s K and V^T with
  // 32-bit byte offsets: seq_len * head_dim * 2 bytes must stay below 2^31.
  if (d->seq_len * (int64_t)d->head_dim * 2 > 0x7fffffff) return RF_ERR_SHAPE;
  if ((int64_t)d->batch * d->heads_q > 65535 || (int64_t)d->batch * d->heads_kv > 65535)
    return RF_ERR_SHAPE;

  RfGeom r;
  memset(&r, 0, sizeof(r));
  r.B = d->batch;
  r.N1 = d->heads_q;
  r.N2 = d->heads_kv;
  r.D = d->head_dim;
  r.G = d->heads_q / d->heads_kv;
  r.layout = d->layout;
  r.S = d->seq_len;

  const bool no_grid = d->grid_t == 0 && d->grid_h == 0 && d->grid_w == 0;
  int64_t n_sparse = 0;
  if (!no_grid) {
    if (d->grid_t <= 0 || d->grid_h <= 0 || d->grid_w <= 0) return RF_ERR_GEOMETRY;
    if (d->prefix_len < 0) return RF_ERR_GEOMETRY;
    const int64_t video = (int64_t)d->grid_t * d->grid_h * d->grid_w;
    if (d->prefix_len + video != d->seq_len) return RF_ERR_GEOMETRY;
    const int64_t frame = (int64_t)d->grid_h * d->grid_w;
    if (d->first_frame_rows != 0 && d->first_frame_rows != frame) return RF_ERR_GEOMETRY;
    r.P = d->prefix_len;
    r.T = d->grid_t;
    r.H = d->grid_h;
    r.W = d->grid_w;
    r.f0 = d->first_frame_rows ? 1 : 0;
    r.pairs = (r.T - r.f0) / 2;
    r.tiles_h = r.H / 8;
    r.tiles_w = r.W / 8;
    n_sparse = (int64_t)r.pairs * r.tiles_h * r.tiles_w;
  }
  const int32_t min_blocks = d->min_sparse_blocks > 0 ? d->min_sparse_blocks : 32;
  r.fallback = (no_grid || d->sparsity == 0.0 || n_sparse < min_blocks) ? 1 : 0;
  if (r.fallback) {
    r.P = r.S;
    r.HF = r.S;
    r.f0 = 0;
    r.pairs = 0;
    r.n_sparse = 0;
    r.U = 0;
    r.prom_per_frame = 0;
    r.n_head = (int32_t)((r.S + 127) / 128);
    r.n_tail = 0;
    r.topk = 0;
  } else {
    if (n_sparse > RF_MAX_SPARSE_BLOCKS) return RF_ERR_UNSUPPORTED;
    const int64_t F = r.f0 ? (int64_t)r.H * r.W : 0;
    r.HF = r.P + F;
    r.n_sparse = (int32_t)n_sparse;
    r.U = (int64_t)r.T * r.H * r.W - F - 128 * n_sparse;
    r.prom_per_frame = (int64_t)r.H * r.W - (int64_t)(8 * r.tiles_h) * (8 * r.tiles_w);
    r.n_head = (int32_t)((r.HF + 127) / 128);
    r.n_tail = (int32_t)((r.U + 127) / 128);
    r.topk = r.n_sparse - (int32_t)floor(d->sparsity * (double)r.n_sparse + 1e-6);
  }
  r.n_blocks = r.n_head + r.n_sparse + r.n_tail;

  if (g) *g = r;
  if (info) {
    memset(info, 0, sizeof(*info));
    info->dense_fallback = r.fallback;
    info->n_blocks = r.n_blocks;
    info->n_head = r.n_head;
    info->n_sparse = r.n_sparse;
    info->n_tail = r.n_tail;
    info->topk = r.topk;
    info->max_kv_blocks = r.n_blocks;
    info->select_rows = r.B * r.n_blocks;
    info->head_rows = r.HF;
    info->sparse_rows = (int64_t)r.n_sparse * 128;
    info->promoted_rows = r.U;
    info->qp_elems = (int64_t)r.B * r.N1 * r.S * r.D;
    info->kp_elems = (int64_t)r.B * r.N2 * r.S * r.D;
    info->vpt_elems = (int64_t)r.B * r.N2 * r.n_blocks * r.D * 128;
    info->q_pool_elems = (int64_t)r.B * r.N1 * r.n_sparse * r.D;
    info->k_pool_elems = (int64_t)r.B * r.N2 * r.n_sparse * r.D;
    info->q_scale_elems = (int64_t)r.B * r.N1 * r.n_blocks;
    info->k_scale_elems = (int64_t)r.B * r.N2 * r.n_blocks;
    info->v_scale_elems = (int64_t)r.B * r.N2 * r.n_blocks;
    info->ws_select_bytes =
        r.fallback ? 0 : rf_ws_scores_bytes(r) + rf_ws_qpool_bytes(r) + rf_ws_kpool_bytes(r);
    info->kp_bytes = 2 * info->kp_elems;
    switch (d->precision) {
      case RF_PREC_BF16:
        info->vpt_bytes = 2 * info->vpt_elems;
        break;
      case RF_PREC_MIX:
      case RF_PREC_FP8:
        info->q8_bytes = info->qp_elems;
        info->k8_bytes = info->kp_elems;
        info->vpt_bytes = (d->precision == RF_PREC_FP8 ? 1 : 2) * info->vpt_elems;
        info->q_scale_bytes = 4 * info->q_scale_elems;
        info->k_scale_bytes = 4 * info->k_scale_elems;
        info->v_scale_bytes = d->precision == RF_PREC_FP8 ? 4 * info->v_scale_elems : 0;
        break;
      default:  // RF_PREC_MXFP4
        info->q8_bytes = info->qp_elems / 2;
        info->k8_bytes = info->kp_elems / 2;
        info->vpt_bytes = info->vpt_elems / 2;
        info->q_scale_bytes = info->qp_elems / 32;
        info->k_scale_bytes = info->kp_elems / 32;
        info->v_scale_bytes = (int64_t)r.B * r.N2 * r.n_blocks * 4 * r.D;
        break;
    }
  }
  return RF_OK;
}

extern "C" {

rf_status rf_plan(const rf_desc* desc, rf_plan_info* info) {
  if (!info) return RF_ERR_NULL;
  return rf_derive(desc, nullptr, info);
}

rf_status rf_permute(const rf_desc* desc, const void* q, const void* k, const void* v, void* qp,
                     void* kp, void* vpt, float* q_pool, float* k_pool, uint8_t* q8, uint8_t* k8,
                     void* q_scale, void* k_scale, void* v_scale, void* stream) {
  RfGeom g;
  rf_plan_info pi;
  rf_status s = rf_derive(desc, &g, &pi);
  if (s != RF_OK) return s;
  if (mxfp4_off(desc)) return RF_ERR_UNSUPPORTED;
  const bool qk8 = desc->precision != RF_PREC_BF16;  // quantised Q/K (codes + scales)
  const bool v8 = desc->precision == RF_PREC_FP8 ||  // quantised V (codes + scales)
                  desc->precision == RF_PREC_MXFP4;
  // Each given input needs somewhere to go.
  if (q && !qp && !q_pool && !(qk8 && q8)) return RF_ERR_NULL;
  if (k && !kp && !k_pool && !(qk8 && k8)) return RF_ERR_NULL;
  if (v && !vpt) return RF_ERR_NULL;
  if (qk8 && ((q && (!q8 || !q_scale)) || (k && (!k8 || !k_scale)))) return RF_ERR_PRECISION;
  if (v8 && v && !v_scale) return RF_ERR_PRECISION;
  const size_t qb = (size_t)pi.qp_elems * 2, kb = (size_t)pi.kp_bytes;
  const size_t vb = (size_t)pi.kp_elems * 2;
  const void* ins[3] = {q, k, v};
  const size_t insz[3] = {qb, vb, vb};
  const void* outs[10] = {qp, kp, vpt, q_pool, k_pool, q8, k8, q_scale, k_scale, v_scale};
  const size_t outsz[10] = {qb, kb, (size_t)pi.vpt_bytes,
                            (size_t)pi.q_pool_elems * 4, (size_t)pi.k_pool_elems * 4,
                            (size_t)pi.q8_bytes, (size_t)pi.k8_bytes,
                            (size_t)pi.q_scale_bytes, (size_t)pi.k_scale_bytes,
                            (size_t)pi.v_scale_bytes};
  for (int i = 0; i < 3; ++i)
    for (int o = 0; o < 10; ++o)
      if (overlaps(ins[i], insz[i], outs[o], outsz[o])) return RF_ERR_ALIAS;
  if (!q && !k && !v) return RF_OK;
  return rf_launch_permute(g, desc->precision, q, k, v, qp, kp, vpt, g.fallback ? nullptr : q_pool,
                           g.fallback ? nullptr : k_pool, qk8 ? q8 : nullptr, qk8 ? k8 : nullptr,
                           qk8 ? q_scale : nullptr, qk8 ? k_scale : nullptr,
                           v8 ? v_scale : nullptr, stream);
}

// Checks shared by rf_pool_select and rf_pool_select_noalloc: the lists are
// present and wide enough, the inputs the call reads are present, and no
// output (lists, and the workspace when the caller gives one) overlaps an
// input or another output.
static rf_status pool_select_operands(const RfGeom& g, const rf_plan_info& pi, const void* qp,
                                      const void* kp, const float* q_pool, const float* k_pool,
                                      const int32_t* select_idx, const int32_t* select_num,
                                      int32_t max_kv, const void* ws, size_t ws_bytes) {
  if (!select_idx || !select_num) return RF_ERR_NULL;
  if (max_kv < g.n_blocks) return RF_ERR_SHAPE;
  const size_t ib = (size_t)pi.select_rows * g.N1 * (size_t)max_kv * 4;
  const size_t nb = (size_t)pi.select_rows * g.N1 * 4;
  if (overlaps(select_idx, ib, select_num, nb)) return RF_ERR_ALIAS;
  if (g.fallback) return RF_OK;  // only the all-dense lists are written
  if ((!q_pool && !qp) || (!k_pool && !kp)) return RF_ERR_NULL;
  // Inputs the call reads: the pooled blocks, or the rows they are pooled from.
  const void* ins[2] = {q_pool ? (const void*)q_pool : qp, k_pool ? (const void*)k_pool : kp};
  const size_t insz[2] = {q_pool ? (size_t)pi.q_pool_elems * 4 : (size_t)pi.qp_elems * 2,
                          k_pool ? (size_t)pi.k_pool_elems * 4 : (size_t)pi.kp_elems * 2};
  const void* outs[3] = {select_idx, select_num, ws};
  const size_t outsz[3] = {ib, nb, ws_bytes};
  for (int i = 0; i < 2; ++i)
    for (int o = 0; o < 3; ++o)
      if (overlaps(ins[i], insz[i], outs[o], outsz[o])) return RF_ERR_ALIAS;
  if (overlaps(ws, ws_bytes, select_idx, ib) || overlaps(ws, ws_bytes, select_num, nb))
    return RF_ERR_ALIAS;
  return RF_OK;
}

rf_status rf_pool_select(const rf_desc* desc, const void* qp, const void* kp, const float* q_pool,
                         const float* k_pool, int32_t* select_idx, int32_t* select_num,
                         int32_t max_kv, void* workspace, size_t workspace_bytes, void* stream) {
  RfGeom g;
  rf_plan_info pi;
  rf_status s = rf_derive(desc, &g, &pi);
  if (s != RF_OK) return s;
  if (!g.fallback) {
    if (!workspace) return RF_ERR_NULL;
    if (workspace_bytes < pi.ws_select_bytes) return RF_ERR_WORKSPACE;
  }
  // The part of the workspace the call writes.
  s = pool_select_operands(g, pi, qp, kp, q_pool, k_pool, select_idx, select_num, max_kv,
                           workspace, rf_ws_used_bytes(g, q_pool != nullptr, k_pool != nullptr));
  if (s != RF_OK) return s;
  return rf_launch_pool_select(g, desc->scale, qp, kp, q_pool, k_pool, select_idx, select_num,
                               max_kv, workspace, stream);
}

rf_status rf_pool_select_noalloc(const rf_desc* desc, const void* qp, const void* kp,
                                 const float* q_pool, const float* k_pool, int32_t* select_idx,
                                 int32_t* select_num, int32_t max_kv, void* stream) {
  RfGeom g;
  rf_plan_info pi;
  rf_status s = rf_derive(desc, &g, &pi);
  if (s != RF_OK) return s;
  s = pool_select_operands(g, pi, qp, kp, q_pool, k_pool, select_idx, select_num, max_kv,
                           nullptr, 0);
  if (s != RF_OK) return s;
  if (rf_ws_used_bytes(g, q_pool != nullptr, k_pool != nullptr) > RF_NOALLOC_SCRATCH_BYTES)
    return RF_ERR_SCRATCH;
  void* ws = nullptr;
  if (!g.fallback) {
    s = rf_noalloc_scratch(&ws);
    if (s != RF_OK) return s;
  }
  return rf_launch_pool_select(g, desc->scale, qp, kp, q_pool, k_pool, select_idx, select_num,
                               max_kv, ws, stream);
}

// Operand checks shared by the two attention entry points: the buffers the
// precision reads are present, and the output overlaps none of them.
static rf_status attn_operands(const rf_desc* desc, const RfGeom& g, const rf_plan_info& pi,
                               const void* qp, const void* kp, const void* vpt, const uint8_t* q8,
                               const uint8_t* k8, const void* q_scale, const void* k_scale,
                               const void* v_scale, const void* out_p) {
  if (!vpt || !out_p) return RF_ERR_NULL;
  const bool qk8 = desc->precision != RF_PREC_BF16;
  const bool v8 = desc->precision == RF_PREC_FP8 || desc->precision == RF_PREC_MXFP4;
  if (qk8) {
    if (!q8 || !k8 || !q_scale || !k_scale) return RF_ERR_PRECISION;
    if (v8 && !v_scale) return RF_ERR_PRECISION;
  } else if (!qp || !kp) {
    return RF_ERR_NULL;
  }
  const size_t ob = (size_t)pi.qp_elems * 2;
  if ((!qk8 && (overlaps(out_p, ob, qp, ob) || overlaps(out_p, ob, kp, (size_t)pi.kp_bytes))) ||
      overlaps(out_p, ob, vpt, (size_t)pi.vpt_bytes) ||
      (qk8 && (overlaps(out_p, ob, q8, (size_t)pi.q8_bytes) ||
               overlaps(out_p, ob, k8, (size_t)pi.k8_bytes) ||
               overlaps(out_p, ob, q_scale, (size_t)pi.q_scale_bytes) ||
               overlaps(out_p, ob, k_scale, (size_t)pi.k_scale_bytes))) ||
      (v8 && overlaps(out_p, ob, v_scale, (size_t)pi.v_scale_bytes)))
    return RF_ERR_ALIAS;
  (void)g;
  return RF_OK;
}

rf_status rf_sparse_attn(const rf_desc* desc, const void* qp, const void* kp, const void* vpt,
                         const uint8_t* q8, const uint8_t* k8, const void* q_scale,
                         const void* k_scale, const void* v_scale, const int32_t* select_idx,
                         const int32_t* select_num, int32_t max_kv, void* out_p, void* stream) {
  RfGeom g;
  rf_plan_info pi;
  rf_status s = rf_derive(desc, &g, &pi);
  if (s != RF_OK) return s;
  if (mxfp4_off(desc)) return RF_ERR_UNSUPPORTED;
  if (!select_idx || !select_num) return RF_ERR_NULL;
  if (max_kv < 1) return RF_ERR_SHAPE;
  s = attn_operands(desc, g, pi, qp, kp, vpt, q8, k8, q_scale, k_scale, v_scale, out_p);
  if (s != RF_OK) return s;
  const size_t ob = (size_t)pi.qp_elems * 2;
  if (overlaps(out_p, ob, select_idx, (size_t)pi.select_rows * g.N1 * (size_t)max_kv * 4) ||
      overlaps(out_p, ob, select_num, (size_t)pi.select_rows * g.N1 * 4))
    return RF_ERR_ALIAS;
  return rf_launch_sparse_attn(g, desc->precision, desc->scale, qp, kp, vpt, q8, k8, q_scale,
                               k_scale, v_scale, select_idx, select_num, max_kv, out_p, stream);
}

rf_status rf_dense_attn(const rf_desc* desc, const void* qp, const void* kp, const void* vpt,
                        const uint8_t* q8, const uint8_t* k8, const void* q_scale,
                        const void* k_scale, const void* v_scale, void* out_p, void* stream) {
  RfGeom g;
  rf_plan_info pi;
  rf_status s = rf_derive(desc, &g, &pi);
  if (s != RF_OK) return s;
  if (mxfp4_off(desc)) return RF_ERR_UNSUPPORTED;
  s = attn_operands(desc, g, pi, qp, kp, vpt, q8, k8, q_scale, k_scale, v_scale, out_p);
  if (s != RF_OK) return s;
  // No lists: the kernel walks every block of the head in order.
  return rf_launch_sparse_attn(g, desc->precision, desc->scale, qp, kp, vpt, q8, k8, q_scale,
                               k_scale, v_scale, nullptr, nullptr, g.n_blocks, out_p, stream);
}

rf_status rf_unpermute(const rf_desc* desc, const void* out_p, void* out, void* stream) {
  RfGeom g;
  rf_plan_info pi;
  rf_status s = rf_derive(desc, &g, &pi);
  if (s != RF_OK) return s;
  if (!out_p || !out) return RF_ERR_NULL;
  if (overlaps(out_p, (size_t)pi.qp_elems * 2, out, (size_t)pi.qp_elems * 2)) return RF_ERR_ALIAS;
  return rf_launch_unpermute(g, out_p, out, stream);
}

const char* rf_status_str(rf_status status) {
  switch (status) {
    case RF_OK: return "ok";
    case RF_ERR_NULL: return "a required pointer is NULL";
    case RF_ERR_LAYOUT: return "layout must be BNSD or TND";
    case RF_ERR_DTYPE: return "element type must be bf16";
    case RF_ERR_SHAPE: return "batch, heads, head_dim, seq_len, scale or max_kv out of range";
    case RF_ERR_BLOCK_SHAPE: return "block shape entries must be positive";
    case RF_ERR_GQA: return "heads_q must be a multiple of heads_kv";
    case RF_ERR_SPARSITY: return "sparsity must be finite and in [0, 1]";
    case RF_ERR_GEOMETRY: return "video grid, prefix or first-frame rows inconsistent with seq_len";
    case RF_ERR_WORKSPACE: return "workspace smaller than rf_plan requires";
    case RF_ERR_UNSUPPORTED: return "valid but not supported by the library (block shape 128x128, "
                                    "head_dim 64/128, <= 8192 sparse blocks)";
    case RF_ERR_PRECISION: return "unknown precision, or a buffer that precision needs is NULL";
    case RF_ERR_HIP: return "HIP launch failed";
    case RF_ERR_ALIAS: return "an output buffer overlaps an input buffer";
    case RF_ERR_SCRATCH: return "the call needs more scratch than rf_pool_select_noalloc's fixed "
                                "device array holds (RF_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

const char* rf_version(void) { return "rf-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"
