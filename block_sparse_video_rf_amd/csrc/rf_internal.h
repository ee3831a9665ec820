// Internal declarations shared by the host plan and the HIP kernels.
//
// RfGeom is the derived per-call geometry, passed by value to every kernel.
// Its meaning follows include/rf.h: permuted order = head segment (prefix +
// first frame), sparse segment (n_sparse blocks of 2 frames x 8x8 tokens),
// promoted tail; blocks of 128 rows with a short last block in the head and
// tail segments.
#pragma once

#include <stdint.h>

#include "rf.h"

#if defined(__HIPCC__)
#define RF_HD __host__ __device__ __forceinline__
#else
#define RF_HD inline
#endif

struct RfGeom {
  int32_t B, N1, N2, D, G;     // batch, query heads, kv heads, head dim, N1 / N2
  int32_t layout;              // rf_layout of the caller's tensors
  int32_t fallback;            // 1: identity arrangement, every block dense
  int64_t S;                   // rows per batch item
  int64_t P;                   // prefix rows
  int64_t HF;                  // head rows: P + first frame (S on fallback)
  int32_t T, H, W;             // latent grid
  int32_t f0;                  // 1 if the first frame is the sink
  int32_t pairs;               // frame pairs cut into boxes
  int32_t tiles_h, tiles_w;    // H / 8, W / 8
  int32_t n_head, n_sparse, n_tail, n_blocks;
  int32_t topk;
  int64_t U;                   // promoted rows
  int64_t prom_per_frame;      // promoted rows of one paired frame: H*W - (8*tiles_h)*(8*tiles_w)
};

// Rows of block j: first permuted row and length (1..128). Head blocks tile
// [0, HF); every later block (sparse segment, then tail) starts at
// HF + 128 (j - n_head) and ends at most at S (S = HF + 128 n_sparse + U, so
// sparse blocks are always whole). Written without branches: kernels call it
// per listed block.
RF_HD void rf_block_rows(const RfGeom& g, int32_t j, int64_t* row0, int32_t* len) {
  const bool head = j < g.n_head;
  const int64_t r0 = head ? (int64_t)j * 128 : g.HF + (int64_t)(j - g.n_head) * 128;
  const int64_t n = (head ? g.HF : g.S) - r0;
  *row0 = r0;
  *len = (int32_t)(n < 128 ? n : 128);
}

// MXFP4 block exponent ("MXAttention: Data-Free Optimal Scaling and
// Pre-Normalization Quantization for MXFP4 Attention", abstract: power-of-two
// scales with the boundary Qmax = 7.25): the smallest e with
// amax <= 7.25 * 2^e, clamped to the E8M0 range [-127, 127]. With
// amax = m * 2^E, m in [1, 2), and 7.25 = 1.8125 * 2^2: e = E - 2 if
// m <= 1.8125, else E - 1 -- exact, from the bits. Zero and subnormal maxima
// (below 2^-126 < 7.25 * 2^-127) give -127. amax is finite and >= 0.
RF_HD int rf_mx_scale_exp(float amax) {
  uint32_t u;
  __builtin_memcpy(&u, &amax, sizeof(u));
  const int eb = (int)(u >> 23);
  if (eb == 0) return -127;
  const int e = eb - 129 + ((u & 0x7fffffu) > 0x680000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Natural row of the token at permuted row r (0 <= r < S).
RF_HD int64_t rf_natural_row(const RfGeom& g, int64_t r) {
  if (r < g.HF) return r;  // prefix and first frame keep their order
  int64_t r2 = r - g.HF;
  const int64_t sparse_rows = (int64_t)g.n_sparse * 128;
  if (r2 < sparse_rows) {
    int32_t blk = (int32_t)(r2 >> 7), in = (int32_t)(r2 & 127);
    int32_t per_pair = g.tiles_h * g.tiles_w;
    int32_t pair = blk / per_pair, rem = blk - pair * per_pair;
    int32_t ti = rem / g.tiles_w, tj = rem - ti * g.tiles_w;
    int32_t t = g.f0 + 2 * pair + (in >> 6);
    int32_t h = 8 * ti + ((in >> 3) & 7);
    int32_t w = 8 * tj + (in & 7);
    return g.P + ((int64_t)t * g.H + h) * g.W + w;
  }
  int64_t u = r2 - sparse_rows;  // rank among promoted rows, natural order
  const int64_t paired_prom = 2 * (int64_t)g.pairs * g.prom_per_frame;
  if (u < paired_prom) {
    int64_t f = u / g.prom_per_frame, m = u - f * g.prom_per_frame;
    int32_t t = g.f0 + (int32_t)f;
    int32_t h8 = 8 * g.tiles_h, w8 = 8 * g.tiles_w, wr = g.W - w8;
    int32_t h, w;
    if (m < (int64_t)h8 * wr) {  // right-hand columns of the tiled rows
      h = (int32_t)(m / wr);
      w = w8 + (int32_t)(m - (int64_t)h * wr);
    } else {                     // whole rows below the tiled rows
      int64_t m2 = m - (int64_t)h8 * wr;
      h = h8 + (int32_t)(m2 / g.W);
      w = (int32_t)(m2 - (int64_t)(h - h8) * g.W);
    }
    return g.P + ((int64_t)t * g.H + h) * g.W + w;
  }
  // Frames after the last pair (an unpaired last frame): natural order.
  return g.P + (int64_t)(g.f0 + 2 * g.pairs) * g.H * g.W + (u - paired_prom);
}

// Element offset of row `s` of (batch b, head n) in the caller's layout.
RF_HD int64_t rf_row_offset(const RfGeom& g, int32_t layout, int32_t heads, int32_t b, int32_t n,
                            int64_t s) {
  if (layout == RF_LAYOUT_TND) return (((int64_t)b * g.S + s) * heads + n) * g.D;
  return (((int64_t)b * heads + n) * g.S + s) * g.D;
}

// Host side: validate a descriptor and derive the geometry (rf_plan.cpp).
rf_status rf_derive(const rf_desc* d, RfGeom* g, rf_plan_info* info);

// Launchers (one per .hip file).
rf_status rf_launch_permute(const RfGeom& g, int32_t precision, const void* q, const void* k,
                            const void* v, void* qp, void* kp, void* vpt, float* q_pool,
                            float* k_pool, uint8_t* q8, uint8_t* k8, void* q_scale,
                            void* k_scale, void* v_scale, void* stream);
rf_status rf_launch_unpermute(const RfGeom& g, const void* out_p, void* out, void* stream);
rf_status rf_launch_pool_select(const RfGeom& g, float scale, const void* qp, const void* kp,
                                const float* q_pool, const float* k_pool, int32_t* select_idx,
                                int32_t* select_num, int32_t max_kv, void* ws, void* stream);
// Device address of rf_pool_select_noalloc's fixed array on the current
// device (looked up once per device; rf_select.hip).
rf_status rf_noalloc_scratch(void** ptr);
rf_status rf_launch_sparse_attn(const RfGeom& g, int32_t precision, float scale, const void* qp,
                                const void* kp, const void* vpt, const uint8_t* q8,
                                const uint8_t* k8, const void* q_scale, const void* k_scale,
                                const void* v_scale, const int32_t* select_idx,
                                const int32_t* select_num, int32_t max_kv, void* out_p,
                                void* stream);

// Workspace layout of rf_pool_select (bytes, 256-aligned pieces):
// scores [B, N1, nS, nS] f32, then q_pool [B, N1, nS, D] f32, then k_pool [B, N2, nS, D] f32.
inline size_t rf_align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t rf_ws_scores_bytes(const RfGeom& g) {
  return rf_align256((size_t)g.B * g.N1 * g.n_sparse * g.n_sparse * 4);
}
inline size_t rf_ws_qpool_bytes(const RfGeom& g) {
  return rf_align256((size_t)g.B * g.N1 * g.n_sparse * g.D * 4);
}
inline size_t rf_ws_kpool_bytes(const RfGeom& g) {
  return rf_align256((size_t)g.B * g.N2 * g.n_sparse * g.D * 4);
}
// Bytes of that workspace a call actually uses: the scores, and the pool
// pieces (in layout order) up to the last one it recomputes.
inline size_t rf_ws_used_bytes(const RfGeom& g, bool have_q_pool, bool have_k_pool) {
  if (g.fallback) return 0;
  size_t n = rf_ws_scores_bytes(g);
  if (!have_q_pool || !have_k_pool) n += rf_ws_qpool_bytes(g);
  if (!have_k_pool) n += rf_ws_kpool_bytes(g);
  return n;
}

// Largest n_sparse the selection kernel holds in LDS.
#define RF_MAX_SPARSE_BLOCKS 8192
