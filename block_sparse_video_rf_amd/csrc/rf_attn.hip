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

constexpr int kThreads8 = 512;  // attention workgroup: 8 waves
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

// The hardware hands workgroup i to XCD i % 8 (MI355X has 8 XCDs, each with
// its own L2). Remap so that every XCD works through one contiguous run of
// the logical work list: neighbouring query blocks of the same head then run
// on the same XCD at the same time and share that XCD's L2 for their key and
// value blocks (they select largely the same ones).
constexpr int32_t kXcds = 8;
__device__ __forceinline__ int32_t xcd_contiguous(int32_t i, int32_t total) {
  const int32_t x = i % kXcds, k = i / kXcds;
  const int32_t q = total / kXcds, r = total % kXcds;
  return x * q + (x < r ? x : r) + k;
}

// Workgroup -> (batch, query block, head). Query blocks that list every key
// block (head and tail segments) run first, so the long workgroups do not
// trail at the end of the grid; each phase is ordered head-major and spread
// over the XCDs in contiguous runs.
__device__ __forceinline__ void decode_wg(const RfGeom& g, int32_t w, int32_t* b, int32_t* q,
                                          int32_t* n) {
  const int32_t n_dense = g.n_head + g.n_tail;
  const int32_t dense_wgs = g.B * g.N1 * n_dense;
  int32_t bn;
  if (w < dense_wgs) {
    const int32_t l = xcd_contiguous(w, dense_wgs);
    bn = l / n_dense;
    const int32_t qd = l - bn * n_dense;
    *q = qd < g.n_head ? qd : qd + g.n_sparse;
  } else {
    const int32_t l = xcd_contiguous(w - dense_wgs, g.B * g.N1 * g.n_sparse);
    bn = l / g.n_sparse;
    *q = g.n_head + (l - bn * g.n_sparse);
  }
  *b = bn / g.N1;
  *n = bn - *b * g.N1;
}

// Scalar (constant address space) view of the list: uniform reads become
// s_load, which neither waits on nor is waited on by the tile prefetches.
typedef const int32_t __attribute__((address_space(4)))* list_ptr;

// Next list position >= it holding a valid block id (or cnt). Uniform.
__device__ __forceinline__ int next_valid(list_ptr list, int it, int cnt, int32_t nb) {
  while (it < cnt) {
    const int32_t j = list[it];
    if (j >= 0 && j < nb) break;
    ++it;
  }
  return it;
}

// Workgroup of 8 waves per (batch, query block, head). Wave w owns query rows
// [32 rg, 32 rg + 32) with rg = w % 4 and key rows [64 kh, 64 kh + 64) of every
// listed block with kh = w / 4: each wave keeps its own running max / sum /
// O^T over its half of the keys, and the two halves are merged through LDS at
// the end (exact: the merge rescales both to the common maximum). Two waves
// per SIMD from one workgroup let one wave's softmax overlap the other's MFMA.
//
// The next block's K and V^T tiles are fetched into registers while the
// current block is computed, then written to LDS between two barriers: the
// global-memory latency hides behind a whole block of work.
template <int D, bool MIX>
__global__ __launch_bounds__(kThreads8, 1) void sparse_attn_kernel(AttnArgs a) {
  constexpr int KSTR = MIX ? D + 16 : 2 * D + 16;  // K row stride in LDS (bytes, padded)
  constexpr int VSTR = 256 + 16;                   // V^T row stride in LDS (bytes, padded)
  constexpr int DT = D / 32;                       // 32-wide channel tiles of O^T
  constexpr int KCH = (MIX ? D : 2 * D) / 16;      // 16-byte chunks per K row
  constexpr int K_PER_T = 128 * KCH / kThreads8;   // K chunks staged per thread
  constexpr int V_PER_T = D * 16 / kThreads8;      // V^T chunks staged per thread
  constexpr int TILE_BYTES = 128 * KSTR + D * VSTR;
  constexpr int MERGE_BYTES = 4 * (DT * 16 + 2) * 64 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[TILE_BYTES > MERGE_BYTES ? TILE_BYTES : MERGE_BYTES];
  uint8_t* ks = smem;
  uint8_t* vs = smem + 128 * KSTR;

  const RfGeom& g = a.g;
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, li = lane % 32, h = lane / 32;
  const int rg = wave & 3, kh = wave >> 2;
  int32_t b, q, n;
  decode_wg(g, blockIdx.x, &b, &q, &n);
  const int32_t nk = n / g.G;
  int64_t row0;
  int32_t len;
  rf_block_rows(g, q, &row0, &len);
  const int qrow = 32 * rg + li;
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
  const list_ptr list = (list_ptr)(a.select_idx + sel_row * a.max_kv);
  int32_t cnt = ((list_ptr)a.select_num)[sel_row];
  cnt = cnt < 0 ? 0 : (cnt > a.max_kv ? a.max_kv : cnt);

  const uint8_t* kbytes =
      MIX ? a.k8 + ((int64_t)b * g.N2 + nk) * g.S * D
          : reinterpret_cast<const uint8_t*>(a.kp + ((int64_t)b * g.N2 + nk) * g.S * D);
  const uint8_t* vbytes = reinterpret_cast<const uint8_t*>(
      a.vpt + ((int64_t)b * g.N2 + nk) * g.n_blocks * (int64_t)D * 128);
  const float* kscale = MIX ? a.k_scale + ((int64_t)b * g.N2 + nk) * g.n_blocks : nullptr;

  // Register staging of one block's K rows and V^T rows. Rows past a short
  // block's end re-read its last row (always in bounds, no branch); they are
  // masked out of the softmax.
  // (Named registers rather than arrays: they must never live in scratch.)
  static_assert(K_PER_T >= 1 && K_PER_T <= 4 && V_PER_T >= 1 && V_PER_T <= 4, "staging size");
  uint4 k0, k1, k2, k3, v0, v1, v2, v3;
#define RF_KLD(VAR, M)                                                                     \
  if constexpr ((M) < K_PER_T) {                                                           \
    const int slot_ = (M) * kThreads8 + tid, r_ = slot_ / KCH, c_ = slot_ % KCH;           \
    const int rr_ = r_ < flen_ ? r_ : flen_ - 1;                                           \
    VAR = *reinterpret_cast<const uint4*>(ksrc_ + rr_ * (MIX ? D : 2 * D) + c_ * 16);      \
  }
#define RF_VLD(VAR, M)                                                                     \
  if constexpr ((M) < V_PER_T) VAR = *reinterpret_cast<const uint4*>(vsrc_ + ((M) * kThreads8 + tid) * 16);
#define RF_FETCH(J)                                                                        \
  do {                                                                                     \
    int64_t fr0_;                                                                          \
    int32_t flen_;                                                                         \
    rf_block_rows(g, (J), &fr0_, &flen_);                                                  \
    const uint8_t* ksrc_ = kbytes + fr0_ * (MIX ? D : 2 * D);                              \
    const uint8_t* vsrc_ = vbytes + (int64_t)(J) * D * 256;                                \
    RF_KLD(k0, 0) RF_KLD(k1, 1) RF_KLD(k2, 2) RF_KLD(k3, 3)                                \
    RF_VLD(v0, 0) RF_VLD(v1, 1) RF_VLD(v2, 2) RF_VLD(v3, 3)                                \
  } while (0)
#define RF_KST(VAR, M)                                                                     \
  if constexpr ((M) < K_PER_T) {                                                           \
    const int slot_ = (M) * kThreads8 + tid, r_ = slot_ / KCH, c_ = slot_ % KCH;           \
    *reinterpret_cast<uint4*>(ks + r_ * KSTR + c_ * 16) = VAR;                             \
  }
#define RF_VST(VAR, M)                                                                     \
  if constexpr ((M) < V_PER_T) {                                                           \
    const int slot_ = (M) * kThreads8 + tid, d_ = slot_ / 16, c_ = slot_ % 16;             \
    *reinterpret_cast<uint4*>(vs + d_ * VSTR + c_ * 16) = VAR;                             \
  }
#define RF_STASH()                                                                         \
  do {                                                                                     \
    RF_KST(k0, 0) RF_KST(k1, 1) RF_KST(k2, 2) RF_KST(k3, 3)                                \
    RF_VST(v0, 0) RF_VST(v1, 1) RF_VST(v2, 2) RF_VST(v3, 3)                                \
  } while (0)

  int it = next_valid(list, 0, cnt, g.n_blocks);
  if (it < cnt) {
    RF_FETCH(list[it]);
    RF_STASH();
  }
  __syncthreads();

  const int krow = 64 * kh + kappa(li);  // this lane's K row in tile t: krow + 32 t
  while (it < cnt) {
    const int32_t j = list[it];
    int64_t kr0;
    int32_t klen;
    rf_block_rows(g, j, &kr0, &klen);
    const int nx = next_valid(list, it + 1, cnt, g.n_blocks);
    // Next block's tiles are in flight during this block's work (the last
    // iteration re-fetches its own block, which nothing reads afterwards).
    RF_FETCH(nx < cnt ? list[nx] : j);

    // S^T tiles: s[t] covers key rows 64 kh + [32t, 32t + 32) of the block.
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) s[t] = f32x16{};
    if constexpr (MIX) {
#pragma unroll
      for (int st = 0; st < QK_STEPS; ++st) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint8_t* kr = ks + (krow + 32 * t) * KSTR + 64 * st + 32 * h;
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
        for (int t = 0; t < 2; ++t) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(ks + (krow + 32 * t) * KSTR +
                                                             32 * st + 16 * h);
          s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[st], s[t], 0, 0, 0);
        }
      }
    }

    // Mask rows past a short block's end.
    if (klen < 128) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kv = 64 * kh + 32 * t + 16 * (v / 8) + 8 * h + (v % 8);
          if (kv >= klen) s[t][v] = -INFINITY;
        }
    }

    float c = a.scale_log2;
    if constexpr (MIX) c *= q_sigma * kscale[j];

    // Maximum over this wave's keys of the row (then the partner half-wave).
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; v += 2) mx = fmaxf(mx, fmaxf(s[t][v], s[t][v + 1]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // The reference maximum m_run only moves when the block exceeds it by more
    // than 8 (log2 units): exponentials stay <= 2^8, which bf16 P and fp32 sums
    // hold as well, and the rescale of O is skipped for most blocks.
    const float mc = mx * c;
    if (__any(mc > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, mc);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < DT; ++e)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[e][v] *= alpha;
    }
    // While every key so far is masked m_run is -inf; any finite stand-in keeps
    // exp2(-inf - m) at 0 instead of NaN.
    const float mneg = -fmaxf(m_run, -1e30f);

    float lsum = 0.0f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[t][8 * u + m], c, mneg));
          lsum += p;
          pf[t][u][m] = (__bf16)p;
        }
    l_run += lsum;

    // O^T += V^T P^T over this wave's 64 key rows (4 k-steps of 16).
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < DT; ++e) {
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(
              vs + (32 * e + li) * VSTR + 2 * (64 * kh + 32 * t + 16 * u + 8 * h));
          o[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[t][u], o[e], 0, 0, 0);
        }

    __syncthreads();  // every wave is done with this block's tiles
    RF_STASH();
    __syncthreads();
    it = nx;
  }

#undef RF_FETCH
#undef RF_STASH
#undef RF_KLD
#undef RF_VLD
#undef RF_KST
#undef RF_VST

  // Merge the two key halves: wave (rg, 1) hands its state to wave (rg, 0).
  float* mbuf = reinterpret_cast<float*>(smem) + rg * (DT * 16 + 2) * 64;
  if (kh == 1) {
#pragma unroll
    for (int e = 0; e < DT; ++e)
#pragma unroll
      for (int v = 0; v < 16; ++v) mbuf[(e * 16 + v) * 64 + lane] = o[e][v];
    mbuf[DT * 16 * 64 + lane] = m_run;
    mbuf[(DT * 16 + 1) * 64 + lane] = l_run;
  }
  __syncthreads();
  if (kh == 1) return;
  const float m1 = mbuf[DT * 16 * 64 + lane];
  const float l1 = mbuf[(DT * 16 + 1) * 64 + lane];
  const float mm = fmaxf(m_run, m1);
  const float a0 = mm == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - mm);
  const float a1 = mm == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - mm);
  float lt = l_run * a0 + l1 * a1;
  lt += __shfl_xor(lt, 32);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (qvalid) {
    uint16_t* orow = a.out_p + (((int64_t)b * g.N1 + n) * g.S + row0 + qrow) * D;
#pragma unroll
    for (int e = 0; e < DT; ++e)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = 32 * e + 8 * a4 + 4 * h;
        __bf16 r[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int v = 4 * a4 + x;
          r[x] = (__bf16)((o[e][v] * a0 + mbuf[(e * 16 + v) * 64 + lane] * a1) * inv);
        }
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
      hipLaunchKernelGGL((sparse_attn_kernel<128, true>), grid, dim3(kThreads8), 0, s, a);
    else
      hipLaunchKernelGGL((sparse_attn_kernel<128, false>), grid, dim3(kThreads8), 0, s, a);
  } else {
    if (mix)
      hipLaunchKernelGGL((sparse_attn_kernel<64, true>), grid, dim3(kThreads8), 0, s, a);
    else
      hipLaunchKernelGGL((sparse_attn_kernel<64, false>), grid, dim3(kThreads8), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? RF_OK : RF_ERR_HIP;
}
