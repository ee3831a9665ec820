// Block-sparse attention: exact softmax(scale * Q K^T) V over the key blocks
// listed in selectIdx ("aclnnRainFusionAttention", Formula; 128 x 128 blocks).
//
// One workgroup of 4 waves per (batch, query block, query head); wave w owns
// query rows [32w, 32w + 32) of the block. The workgroup walks its list of
// key blocks; for each it stages K (row-major, [128][D]) and V (already
// block-transposed by the permute kernel, [D][128]) in LDS, then
//
//   S^T = K Q^T  with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS,
//                B = the wave's Q rows, held in registers for the whole walk)
//   online softmax in fp32, exp2 with the scale folded in
//   O^T += V^T P^T  with the same MFMA (A = V^T rows from LDS, B = P in bf16)
//
// Computing the transposed products makes every lane own one query row
// (column l % 32 of the 32x32 accumulator tiles), so the row maximum, the
// running sum and the rescale of O are lane-local except for one exchange
// with the partner lane l ^ 32 for the maximum.
//
// K rows are fed to the A operand in a permuted order (kappa(), which swaps
// bits 2 and 3 of the tile row) so that the 16 accumulator values of a lane
// in a tile cover key rows 16*(v/8) + 8*(l/32) + v%8: each group of 8 is
// contiguous, which is exactly the 8-value k-slice the PV product wants from
// the B operand, and the matching V^T slice is one contiguous 16-byte LDS
// read.
//
// The mix precision replaces the QK^T operands by fp8 E4M3 codes
// (v_mfma_scale_f32_32x32x64_f8f6f4, unit block scales) and folds
// scale * q_scale * k_scale of the block pair into the exponent multiplier.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "rf_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

struct AttnArgs {
  RfGeom g;
  float scale_log2;  // scale * log2(e)
  const uint16_t* qp;
  const uint16_t* kp;
  const uint16_t* vpt;
  const uint8_t* q8;
  const uint8_t* k8;
  const float* q_scale;
  const float* k_scale;
  const int32_t* select_idx;
  const int32_t* select_num;
  int32_t max_kv;
  uint16_t* out_p;
};

__device__ __forceinline__ int kappa(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Workgroup -> (batch, query block, head). Query blocks that list every key
// block (head and tail segments) run first, so the long workgroups do not
// trail at the end of the grid; within each group consecutive workgroups
// share a head and therefore its K/V.
__device__ __forceinline__ void decode_wg(const RfGeom& g, int32_t w, int32_t* b, int32_t* q,
                                          int32_t* n) {
  const int32_t n_dense = g.n_head + g.n_tail;
  const int32_t dense_wgs = g.B * g.N1 * n_dense;
  int32_t bn;
  if (w < dense_wgs) {
    bn = w / n_dense;
    const int32_t qd = w - bn * n_dense;
    *q = qd < g.n_head ? qd : qd + g.n_sparse;
  } else {
    const int32_t w2 = w - dense_wgs;
    bn = w2 / g.n_sparse;
    *q = g.n_head + (w2 - bn * g.n_sparse);
  }
  *b = bn / g.N1;
  *n = bn - *b * g.N1;
}

template <int D, bool MIX>
__global__ __launch_bounds__(kThreads, 2) void sparse_attn_kernel(AttnArgs a) {
  constexpr int KSTR = MIX ? (D + 16) : (D + 8);  // K row stride in LDS (elements)
  constexpr int VSTR = 128 + 8;                   // V^T row stride in LDS (elements)
  constexpr int DT = D / 32;                      // 32-wide channel tiles of O^T
  typedef typename std::conditional<MIX, uint8_t, uint16_t>::type kelem;
  __shared__ __attribute__((aligned(16))) kelem ks[128 * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vs[D * VSTR];

  const RfGeom& g = a.g;
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, li = lane % 32, h = lane / 32;
  int32_t b, q, n;
  decode_wg(g, blockIdx.x, &b, &q, &n);
  const int32_t nk = n / g.G;
  int64_t row0;
  int32_t len;
  rf_block_rows(g, q, &row0, &len);
  const int qrow = 32 * wave + li;
  const bool qvalid = qrow < len;

  // Q fragment (B operand of S^T = K Q^T): query row qrow, channels by k-step.
  constexpr int QK_STEPS = MIX ? D / 64 : D / 16;
  bf16x8 qf[MIX ? 1 : QK_STEPS];
  i32x8 qf8[MIX ? QK_STEPS : 1];
  float q_sigma = 1.0f;
  if constexpr (MIX) {
    const uint8_t* qr = a.q8 + (((int64_t)b * g.N1 + n) * g.S + row0 + qrow) * D;
#pragma unroll
    for (int st = 0; st < QK_STEPS; ++st) {
      if (qvalid) {
        const uint4 x0 = *reinterpret_cast<const uint4*>(qr + 64 * st + 32 * h);
        const uint4 x1 = *reinterpret_cast<const uint4*>(qr + 64 * st + 32 * h + 16);
        qf8[st] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                        (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      } else {
        qf8[st] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
    q_sigma = a.q_scale[((int64_t)b * g.N1 + n) * g.n_blocks + q];
  } else {
    const uint16_t* qr = a.qp + (((int64_t)b * g.N1 + n) * g.S + row0 + qrow) * D;
#pragma unroll
    for (int st = 0; st < QK_STEPS; ++st) {
      if (qvalid) {
        qf[st] = *reinterpret_cast<const bf16x8*>(qr + 16 * st + 8 * h);
      } else {
        qf[st] = bf16x8{};
      }
    }
  }

  f32x16 o[DT];
#pragma unroll
  for (int e = 0; e < DT; ++e) o[e] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;

  const int64_t sel_row = ((int64_t)b * g.n_blocks + q) * g.N1 + n;
  const int32_t* list = a.select_idx + sel_row * a.max_kv;
  int32_t cnt = a.select_num[sel_row];
  cnt = cnt < 0 ? 0 : (cnt > a.max_kv ? a.max_kv : cnt);

  const int64_t kbase_head = ((int64_t)b * g.N2 + nk) * g.S;
  for (int it = 0; it < cnt; ++it) {
    const int32_t j = list[it];
    if (j < 0 || j >= g.n_blocks) continue;  // same j for the whole workgroup
    int64_t kr0;
    int32_t klen;
    rf_block_rows(g, j, &kr0, &klen);

    __syncthreads();  // previous block's LDS reads are done
    if constexpr (MIX) {
      constexpr int C = D / 16;  // 16-byte chunks per fp8 row
      constexpr int RPP = kThreads / C;
      const int c = tid % C, rs = tid / C;
      const uint8_t* src = a.k8 + (kbase_head + kr0) * D;
#pragma unroll
      for (int p = 0; p < 128 / RPP; ++p) {
        const int r = p * RPP + rs;
        if (r < klen)
          *reinterpret_cast<uint4*>(ks + r * KSTR + c * 16) =
              *reinterpret_cast<const uint4*>(src + (int64_t)r * D + c * 16);
      }
    } else {
      constexpr int C = D / 8;
      constexpr int RPP = kThreads / C;
      const int c = tid % C, rs = tid / C;
      const uint16_t* src = a.kp + (kbase_head + kr0) * D;
#pragma unroll
      for (int p = 0; p < 128 / RPP; ++p) {
        const int r = p * RPP + rs;
        if (r < klen)
          *reinterpret_cast<uint4*>(ks + r * KSTR + c * 8) =
              *reinterpret_cast<const uint4*>(src + (int64_t)r * D + c * 8);
      }
    }
    {
      const uint16_t* vsrc = a.vpt + (((int64_t)b * g.N2 + nk) * g.n_blocks + j) * (int64_t)D * 128;
#pragma unroll
      for (int m = 0; m < D / 16; ++m) {
        const int qd = tid + kThreads * m;
        const int d = qd / 16, cc = qd % 16;
        *reinterpret_cast<uint4*>(vs + d * VSTR + cc * 8) =
            *reinterpret_cast<const uint4*>(vsrc + d * 128 + cc * 8);
      }
    }
    __syncthreads();

    // S^T tiles: s[t] covers key rows [32t, 32t + 32) of the block.
    f32x16 s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) s[t] = f32x16{};
    const int krow = kappa(li);
    if constexpr (MIX) {
#pragma unroll
      for (int st = 0; st < QK_STEPS; ++st) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint8_t* kr = ks + (32 * t + krow) * KSTR + 64 * st + 32 * h;
          const uint4 x0 = *reinterpret_cast<const uint4*>(kr);
          const uint4 x1 = *reinterpret_cast<const uint4*>(kr + 16);
          const i32x8 ka = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                            (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
          s[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qf8[st], s[t], 0, 0, 0, 127,
                                                                 0, 127);
        }
      }
    } else {
#pragma unroll
      for (int st = 0; st < QK_STEPS; ++st) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x8 ka =
              *reinterpret_cast<const bf16x8*>(ks + (32 * t + krow) * KSTR + 16 * st + 8 * h);
          s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[st], s[t], 0, 0, 0);
        }
      }
    }

    // Mask rows past a short block's end.
    if (klen < 128) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kv = 32 * t + 16 * (v / 8) + 8 * h + (v % 8);
          if (kv >= klen) s[t][v] = -INFINITY;
        }
    }

    float c = a.scale_log2;
    if constexpr (MIX) c *= q_sigma * a.k_scale[((int64_t)b * g.N2 + nk) * g.n_blocks + j];

    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[t][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    float lsum = 0.0f;
    bf16x8 pf[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[t][8 * u + m], c, -m_new));
          lsum += p;
          pf[t][u][m] = (__bf16)p;
        }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int e = 0; e < DT; ++e)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[e][v] *= alpha;

    // O^T += V^T P^T over the block's 128 key rows (8 k-steps of 16).
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < DT; ++e) {
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(vs + (32 * e + li) * VSTR + 32 * t +
                                                             16 * u + 8 * h);
          o[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[t][u], o[e], 0, 0, 0);
        }
  }

  const float l = l_run + __shfl_xor(l_run, 32);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if (qvalid) {
    uint16_t* orow = a.out_p + (((int64_t)b * g.N1 + n) * g.S + row0 + qrow) * D;
#pragma unroll
    for (int e = 0; e < DT; ++e)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = 32 * e + 8 * a4 + 4 * h;
        __bf16 r[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) r[x] = (__bf16)(o[e][4 * a4 + x] * inv);
        uint2 w;
        __builtin_memcpy(&w, r, 8);
        *reinterpret_cast<uint2*>(orow + d0) = w;
      }
  }
}

}  // namespace

rf_status rf_launch_sparse_attn(const RfGeom& g, int32_t precision, float scale, const void* qp,
                                const void* kp, const void* vpt, const uint8_t* q8,
                                const uint8_t* k8, const float* q_scale, const float* k_scale,
                                const int32_t* select_idx, const int32_t* select_num,
                                int32_t max_kv, void* out_p, void* stream) {
  AttnArgs a;
  a.g = g;
  a.scale_log2 = scale * kLog2e;
  a.qp = static_cast<const uint16_t*>(qp);
  a.kp = static_cast<const uint16_t*>(kp);
  a.vpt = static_cast<const uint16_t*>(vpt);
  a.q8 = q8;
  a.k8 = k8;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.select_idx = select_idx;
  a.select_num = select_num;
  a.max_kv = max_kv;
  a.out_p = static_cast<uint16_t*>(out_p);
  const int64_t wgs = (int64_t)g.B * g.N1 * g.n_blocks;
  if (wgs > 0x7fffffff) return RF_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((uint32_t)wgs);
  const bool mix = precision == RF_PREC_MIX;
  if (g.D == 128) {
    if (mix)
      hipLaunchKernelGGL((sparse_attn_kernel<128, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((sparse_attn_kernel<128, false>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (mix)
      hipLaunchKernelGGL((sparse_attn_kernel<64, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((sparse_attn_kernel<64, false>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? RF_OK : RF_ERR_HIP;
}
