// Block scoring and top-k selection: builds selectIdx / selectNum.
//
// "RainFusion Attention", introduction: pooled 128-token key blocks are
// ranked per query block and the highest-scoring ones are attended; the
// prefix, the first frame and the promoted tail stay dense. Configuration:
// sparsity is the nominal dropped fraction. "aclnnRainFusionAttention",
// constraints: selectIdx [T, heads, maxKv] with -1 in unused entries and
// selectNum [T, heads], T = batch * query blocks.
//
// Kernels:
//   pool_kernel   (only when the caller has no pooled blocks) mean of each
//                 sparse block of qp / kp, fp32.
//   score_kernel  per (batch, query head): Sc = scale * Qbar Kbar^T over the
//                 sparse blocks, a small fp32 GEMM tiled 64x64 through LDS
//                 (4x4 outputs per thread, fixed summation order over D).
//   select_wave_kernel  one wave per selectIdx row (batch, query block, head),
//                 up to 2048 sparse blocks: dense query blocks write
//                 0..n_blocks-1; sparse ones hold the row's order-preserving
//                 score keys in registers, build the k-th largest key bit by
//                 bit from the top (a bit stays set while at least k keys are
//                 >= the candidate, counted with ballots), keep every key above
//                 it and the lowest-id keys equal to it, and write the
//                 ascending union with the dense blocks.
//   select_kernel the same rule with one workgroup per row and the keys in LDS
//                 (a 4-pass 8-bit radix select), for more sparse blocks.
//   Integer work only after the scores, so the lists are exact for given
//   scores, and both kernels give the same lists.
#include <hip/hip_runtime.h>

#include <mutex>

#include "rf_internal.h"

namespace {

constexpr int kThreads = 256;

struct PoolArgs {
  RfGeom g;
  const uint16_t* qp;
  const uint16_t* kp;
  float* q_pool;
  float* k_pool;
};

template <int D>
__global__ __launch_bounds__(kThreads) void pool_kernel(PoolArgs a) {
  constexpr int C = D / 8, RPP = kThreads / C, PASSES = 128 / RPP;
  __shared__ float red[kThreads * 8];
  const RfGeom& g = a.g;
  const int tid = threadIdx.x, c = tid % C, rsub = tid / C;
  const int32_t js = blockIdx.x;
  int32_t y = blockIdx.y;
  const bool is_q = y < g.B * g.N1;
  if (!is_q) y -= g.B * g.N1;
  const int heads = is_q ? g.N1 : g.N2;
  const uint16_t* src = is_q ? a.qp : a.kp;
  float* dst = is_q ? a.q_pool : a.k_pool;
  if (!src || !dst) return;
  const int32_t b = y / heads, n = y % heads;
  const int64_t row0 = g.HF + (int64_t)js * 128;
  const uint16_t* base = src + (((int64_t)b * heads + n) * g.S + row0) * D;
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const uint4 v = *reinterpret_cast<const uint4*>(base + (int64_t)(p * RPP + rsub) * D + c * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[2 * e] += __uint_as_float(w[e] << 16);
      s[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rsub * D + c * 8 + e] = s[e];
  __syncthreads();
  if (tid < D) {
    float t = 0.0f;
    for (int r = 0; r < RPP; ++r) t += red[r * D + tid];
    dst[(((int64_t)b * heads + n) * g.n_sparse + js) * D + tid] = t * (1.0f / 128.0f);
  }
}

struct ScoreArgs {
  RfGeom g;
  float scale;
  const float* q_pool;  // [B, N1, nS, D]
  const float* k_pool;  // [B, N2, nS, D]
  float* scores;        // [B, N1, nS, nS]
};

// 64x64 output tile per workgroup; D consumed in slices of 32.
__global__ __launch_bounds__(kThreads) void score_kernel(ScoreArgs a) {
  constexpr int TI = 64, TK = 32;
  __shared__ float qs[TK][TI + 4];
  __shared__ float ks[TK][TI + 4];
  const RfGeom& g = a.g;
  const int tid = threadIdx.x;
  const int ti = tid / 16, tj = tid % 16;
  const int i0 = blockIdx.y * TI, j0 = blockIdx.x * TI;
  const int32_t bn = blockIdx.z;
  const int32_t b = bn / g.N1, n = bn % g.N1;
  const int nS = g.n_sparse, D = g.D;
  const float* qb = a.q_pool + ((int64_t)b * g.N1 + n) * nS * D;
  const float* kb = a.k_pool + ((int64_t)b * g.N2 + n / g.G) * nS * D;
  float acc[4][4] = {};
  for (int d0 = 0; d0 < D; d0 += TK) {
    // 64 rows x 32 channels of each operand: 2048 floats, 8 per thread.
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int e = tid + kThreads * m;
      const int r = e / TK, dd = e % TK;
      qs[dd][r] = (i0 + r < nS) ? qb[(int64_t)(i0 + r) * D + d0 + dd] : 0.0f;
      ks[dd][r] = (j0 + r < nS) ? kb[(int64_t)(j0 + r) * D + d0 + dd] : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int dd = 0; dd < TK; ++dd) {
      float x[4], y[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        x[u] = qs[dd][ti * 4 + u];
        y[u] = ks[dd][tj * 4 + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[u][w] = fmaf(x[u], y[w], acc[u][w]);
    }
    __syncthreads();
  }
  float* out = a.scores + (int64_t)bn * nS * nS;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = i0 + ti * 4 + u;
    if (i >= nS) continue;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int j = j0 + tj * 4 + w;
      if (j < nS) out[(int64_t)i * nS + j] = a.scale * acc[u][w];
    }
  }
}

struct SelectArgs {
  RfGeom g;
  const float* scores;
  int32_t* select_idx;
  int32_t* select_num;
  int32_t max_kv;
};

// Order-preserving unsigned key of a float (larger float -> larger key);
// +0 and -0 share a key so that equal scores tie exactly.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f == 0.0f) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan of one int per thread over the workgroup (Hillis-Steele in LDS).
__device__ __forceinline__ int block_inclusive_scan(int x, int* buf) {
  const int tid = threadIdx.x;
  buf[tid] = x;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int t = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += t;
    __syncthreads();
  }
  const int r = buf[tid];
  __syncthreads();
  return r;
}

// Exclusive prefix sum of one int per lane over a wave.
__device__ __forceinline__ int wave_exclusive_scan(int x, int lane) {
  int incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  return incl - x;
}

// One wave per selectIdx row; lane l holds the keys of sparse ids
// [PER l, PER l + PER), so id order is lane-major and then slot order.
template <int PER>
__global__ __launch_bounds__(kThreads) void select_wave_kernel(SelectArgs a) {
  const RfGeom& g = a.g;
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)g.B * g.N1 * g.n_blocks;
  // Rows ordered (batch, head, query block), query block fastest: the waves of
  // a workgroup read neighbouring score rows.
  const int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (r >= rows) return;  // uniform over the wave
  const int32_t q = (int32_t)(r % g.n_blocks);
  const int64_t bn = r / g.n_blocks;
  const int32_t n = (int32_t)(bn % g.N1), b = (int32_t)(bn / g.N1);
  const int64_t row = (int64_t)b * g.n_blocks + q;
  int32_t* out = a.select_idx + (row * g.N1 + n) * a.max_kv;
  const int32_t nB = g.n_blocks;
  const bool sparse_q = q >= g.n_head && q < g.n_head + g.n_sparse;
  if (!sparse_q) {
    for (int p = lane; p < a.max_kv; p += 64) out[p] = p < nB ? p : -1;
    if (lane == 0) a.select_num[row * g.N1 + n] = nB;
    return;
  }
  const int nS = g.n_sparse, k = g.topk;
  const int32_t nh = g.n_head;
  const int count = nh + k + g.n_tail;
  for (int p = lane; p < a.max_kv; p += 64) {
    if (p < nh) out[p] = p;
    else if (p >= nh + k && p < count) out[p] = nh + nS + (p - nh - k);
    else if (p >= count) out[p] = -1;
  }
  if (lane == 0) a.select_num[row * g.N1 + n] = count;
  if (k == 0) return;

  const float* sc = a.scores + (((int64_t)b * g.N1 + n) * nS + (q - nh)) * nS;
  const int i0 = lane * PER;
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) key[i] = i0 + i < nS ? order_key(sc[i0 + i]) : 0u;
  // Finite scores have keys > 0, so the zero keys of unused slots never reach
  // the threshold.
  uint32_t kth = 0;
  int need = k;  // keys equal to kth still to take (lowest ids first)
  if (k < nS) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = kth | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) cnt += __popcll(__ballot(key[i] >= cand));
      if (cnt >= k) kth = cand;
    }
    int gt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) gt += __popcll(__ballot(key[i] > kth));
    need = k - gt;
  }
  int eq = 0;
  if (k < nS) {
#pragma unroll
    for (int i = 0; i < PER; ++i) eq += (i0 + i < nS && key[i] == kth) ? 1 : 0;
  }
  int rank = wave_exclusive_scan(eq, lane);  // ties with lower ids
  bool take[PER];
  int ntake = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    bool t;
    if (i0 + i >= nS) t = false;
    else if (k >= nS || key[i] > kth) t = true;
    else if (key[i] == kth) t = rank++ < need;
    else t = false;
    take[i] = t;
    ntake += t ? 1 : 0;
  }
  int pos = nh + wave_exclusive_scan(ntake, lane);
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (take[i]) out[pos++] = nh + i0 + i;
}

__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a) {
  __shared__ uint32_t keys[RF_MAX_SPARSE_BLOCKS];
  __shared__ int hist[kThreads];
  __shared__ int scan_buf[kThreads];
  __shared__ uint32_t sel_digit;
  __shared__ int sel_need;
  const RfGeom& g = a.g;
  const int tid = threadIdx.x;
  const int32_t q = blockIdx.x, n = blockIdx.y, b = blockIdx.z;
  const int64_t row = (int64_t)b * g.n_blocks + q;
  int32_t* out = a.select_idx + (row * g.N1 + n) * a.max_kv;
  const bool sparse_q = q >= g.n_head && q < g.n_head + g.n_sparse;
  const int32_t nB = g.n_blocks;

  if (!sparse_q) {
    for (int p = tid; p < a.max_kv; p += kThreads) out[p] = p < nB ? p : -1;
    if (tid == 0) a.select_num[row * g.N1 + n] = nB;
    return;
  }

  const int nS = g.n_sparse, k = g.topk;
  const int32_t nh = g.n_head;
  const int count = g.n_head + k + g.n_tail;
  // Head ids, tail ids and the -1 fill.
  for (int p = tid; p < a.max_kv; p += kThreads) {
    if (p < nh) out[p] = p;
    else if (p >= nh + k && p < count) out[p] = nh + nS + (p - nh - k);
    else if (p >= count) out[p] = -1;
  }
  if (tid == 0) a.select_num[row * g.N1 + n] = count;
  if (k == 0) return;

  const float* sc = a.scores + (((int64_t)b * g.N1 + n) * nS + (q - nh)) * nS;
  for (int i = tid; i < nS; i += kThreads) keys[i] = order_key(sc[i]);
  __syncthreads();

  // k-th largest key, 8 bits at a time from the top.
  uint32_t prefix = 0, mask = 0;
  int need = k;  // how many keys matching `prefix` still have to be taken
  if (k < nS) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < nS; i += kThreads) {
        const uint32_t key = keys[i];
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      // Thread t looks at digit 255 - t; cumulative counts from the top digit down.
      const int cnt = hist[255 - tid];
      const int incl = block_inclusive_scan(cnt, scan_buf);
      if (incl >= need && incl - cnt < need) {
        sel_digit = 255u - tid;
        sel_need = need - (incl - cnt);
      }
      __syncthreads();
      prefix |= sel_digit << shift;
      mask |= 255u << shift;
      need = sel_need;
      __syncthreads();
    }
  }
  const uint32_t kth = prefix;

  // Each thread owns a contiguous run of ids, so scans follow id order.
  const int per = (nS + kThreads - 1) / kThreads;
  const int s0 = min(nS, tid * per), s1 = min(nS, s0 + per);
  int eq = 0;
  if (k < nS)
    for (int i = s0; i < s1; ++i) eq += keys[i] == kth;
  const int eq_before = block_inclusive_scan(eq, scan_buf) - eq;
  int take = 0;
  {
    int rank = eq_before;
    for (int i = s0; i < s1; ++i) {
      const uint32_t key = keys[i];
      bool t;
      if (k >= nS) t = true;
      else if (key > kth) t = true;
      else if (key == kth) t = rank++ < need;
      else t = false;
      take += t;
    }
  }
  int pos = nh + block_inclusive_scan(take, scan_buf) - take;
  {
    int rank = eq_before;
    for (int i = s0; i < s1; ++i) {
      const uint32_t key = keys[i];
      bool t;
      if (k >= nS) t = true;
      else if (key > kth) t = true;
      else if (key == kth) t = rank++ < need;
      else t = false;
      if (t) out[pos++] = nh + i;
    }
  }
}

}  // namespace

// Workspace of rf_pool_select_noalloc: a fixed array that every device the
// library runs on holds until the process ends (scores, then recomputed
// pools, as in a caller's workspace). In host code `scratch` names a host-side
// stand-in, never the device memory: host code only uses the address that
// hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) uint8_t scratch[RF_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device id
}  // namespace

rf_status rf_noalloc_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RF_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RF_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return RF_OK;
}

rf_status rf_launch_pool_select(const RfGeom& g, float scale, const void* qp, const void* kp,
                                const float* q_pool, const float* k_pool, int32_t* select_idx,
                                int32_t* select_num, int32_t max_kv, void* ws, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  SelectArgs sa;
  sa.g = g;
  sa.scores = nullptr;
  sa.select_idx = select_idx;
  sa.select_num = select_num;
  sa.max_kv = max_kv;
  if (!g.fallback) {
    char* w = static_cast<char*>(ws);
    float* scores = reinterpret_cast<float*>(w);
    float* qpool_ws = reinterpret_cast<float*>(w + rf_ws_scores_bytes(g));
    float* kpool_ws = reinterpret_cast<float*>(w + rf_ws_scores_bytes(g) + rf_ws_qpool_bytes(g));
    if (!q_pool || !k_pool) {
      PoolArgs pa;
      pa.g = g;
      pa.qp = q_pool ? nullptr : static_cast<const uint16_t*>(qp);
      pa.kp = k_pool ? nullptr : static_cast<const uint16_t*>(kp);
      pa.q_pool = qpool_ws;
      pa.k_pool = kpool_ws;
      const dim3 grid(g.n_sparse, g.B * (g.N1 + g.N2));
      if (g.D == 128)
        hipLaunchKernelGGL(pool_kernel<128>, grid, dim3(kThreads), 0, s, pa);
      else
        hipLaunchKernelGGL(pool_kernel<64>, grid, dim3(kThreads), 0, s, pa);
      if (!q_pool) q_pool = qpool_ws;
      if (!k_pool) k_pool = kpool_ws;
    }
    ScoreArgs ca;
    ca.g = g;
    ca.scale = scale;
    ca.q_pool = q_pool;
    ca.k_pool = k_pool;
    ca.scores = scores;
    const int tiles = (g.n_sparse + 63) / 64;
    hipLaunchKernelGGL(score_kernel, dim3(tiles, tiles, g.B * g.N1), dim3(kThreads), 0, s, ca);
    sa.scores = scores;
  }
  const int64_t rows = (int64_t)g.B * g.N1 * g.n_blocks;
  const dim3 wave_grid((uint32_t)((rows + kThreads / 64 - 1) / (kThreads / 64)));
  if (g.n_sparse <= 512)
    hipLaunchKernelGGL(select_wave_kernel<8>, wave_grid, dim3(kThreads), 0, s, sa);
  else if (g.n_sparse <= 1024)
    hipLaunchKernelGGL(select_wave_kernel<16>, wave_grid, dim3(kThreads), 0, s, sa);
  else if (g.n_sparse <= 2048)
    hipLaunchKernelGGL(select_wave_kernel<32>, wave_grid, dim3(kThreads), 0, s, sa);
  else
    hipLaunchKernelGGL(select_kernel, dim3(g.n_blocks, g.N1, g.B), dim3(kThreads), 0, s, sa);
  return hipGetLastError() == hipSuccess ? RF_OK : RF_ERR_HIP;
}
