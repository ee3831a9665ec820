// Arrangement kernels: permute (+ block-mean pooling, + quantisation of the
// fp8-family and mxfp4 precisions) and the inverse permutation.
//
// "RainFusion Attention" (introduction, Geometry handling) and the xLLM
// pull request "feat: add RainFusion sparse attention for wan2.2" (commit
// summary: frame-pairing rearrange of Q, K and V in one call; inverse
// rearrange; roundtrip check). Block means as representative tokens: the
// RainFusion2.0 abstract, insight 1.
//
// One launch covers Q, K and V: workgroup (block j, slot y) where y runs over
// the B*N1 query heads, then the B*N2 key heads, then the B*N2 value heads.
// A workgroup moves one block (<= 128 rows of D bf16) and never needs a map
// in memory: rf_natural_row() decodes the source row from the geometry. The
// work is a pure HBM stream (read once, write once); every 16-byte chunk is
// one global load and one global store, rows of D*2 bytes are read whole.
//
// V is written block-transposed (vpt[b, n, j, d, c]) so that the attention
// kernel's PV product reads its MFMA operand with contiguous 16-byte LDS
// loads; the transpose goes through LDS here, where the work is bandwidth
// bound anyway.
//
// mxfp4 (OCP MXFP4 with the MXAttention scale rule, abstract: power-of-two
// scales with the boundary 7.25): Q and K rows in blocks of 32 channels, V in
// the 32-key quarters of each block per channel; each block's exponent e is
// the smallest with amax <= 7.25 * 2^e, stored as the E8M0 byte e + 127, and
// its values as E2M1 codes of x / 2^e (nearest even, saturating at 6).
#include <hip/hip_runtime.h>

#include "rf_internal.h"
#include "rf_mx.h"

namespace {

constexpr int kThreads = 256;

struct PermuteArgs {
  RfGeom g;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* qp;
  uint16_t* kp;
  uint16_t* vpt;
  float* q_pool;
  float* k_pool;
  uint8_t* q8;
  uint8_t* k8;
  void* q_scale;  // fp32 per block (mix, fp8) or E8M0 bytes per 32 channels (mxfp4)
  void* k_scale;
  void* v_scale;  // fp8: fp32 power-of-two V scales; mxfp4: E8M0 bytes per key quarter
  int mx;         // mxfp4 precision
};

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// E4M3 codes come from gfx950's v_cvt_pk_fp8_f32 (OCP E4M3, round to nearest
// even). Every input here is finite with magnitude at most 448 (times one
// rounding of the scale), where that conversion is the plain nearest-even
// encoding, -0 giving the sign bit alone.

// Streaming (non-temporal) stores of 16 and 8 bytes: outputs that this kernel
// does not read again.
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_stream(void* p, uint32_t x, uint32_t y, uint32_t z, uint32_t w) {
  __builtin_nontemporal_store(v4u{x, y, z, w}, reinterpret_cast<v4u*>(p));
}
__device__ __forceinline__ void store_stream(void* p, uint32_t x, uint32_t y) {
  __builtin_nontemporal_store(v2u{x, y}, reinterpret_cast<v2u*>(p));
}
// Streaming 16-byte load of an input read exactly once.
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const v4u x = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}

// Smallest e with amax <= 448 * 2^e, clamped to [-126, 127] (a normal fp32
// power of two); 0 for amax == 0. With amax = f * 2^x, f in [0.5, 1), and
// 448 = 0.875 * 2^9: e = x - 9 if f <= 0.875, else x - 8 (exact).
__device__ __forceinline__ int pow2_scale_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  int x;
  const float f = frexpf(amax, &x);
  const int e = f <= 0.875f ? x - 9 : x - 8;
  return e < -126 ? -126 : (e > 127 ? 127 : e);
}

// Block-wide maximum over the 256 threads: a wave reduction by lane shuffles,
// then the four wave maxima through LDS (one barrier). A maximum does not
// depend on the order it is taken in.
__device__ __forceinline__ float block_max(float x, float* red) {
  static_assert(kThreads == 4 * 64, "four waves of 64 lanes");
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) red[tid >> 6] = x;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

template <int D>
__global__ __launch_bounds__(kThreads) void permute_kernel(PermuteArgs a) {
  constexpr int C = D / 8;                 // 16-byte chunks per row
  constexpr int RPP = kThreads / C;        // rows per pass
  constexpr int PASSES = 128 / RPP;
  const RfGeom& g = a.g;
  const int tid = threadIdx.x;
  const int c = tid % C;
  const int rsub = tid / C;
  const int32_t j = blockIdx.x;
  int32_t y = blockIdx.y;

  // Which tensor, batch item and head.
  int kind;  // 0 = Q, 1 = K, 2 = V
  int heads;
  if (y < g.B * g.N1) {
    kind = 0;
    heads = g.N1;
  } else if (y < g.B * (g.N1 + g.N2)) {
    kind = 1;
    y -= g.B * g.N1;
    heads = g.N2;
  } else {
    kind = 2;
    y -= g.B * (g.N1 + g.N2);
    heads = g.N2;
  }
  const int32_t b = y / heads, n = y % heads;
  const uint16_t* src = kind == 0 ? a.q : (kind == 1 ? a.k : a.v);
  if (src == nullptr) return;  // uniform over the workgroup

  int64_t row0;
  int32_t len;
  rf_block_rows(g, j, &row0, &len);

  uint4 val[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int i = p * RPP + rsub;
    if (i < len) {
      const int64_t nat = rf_natural_row(g, row0 + i);
      val[p] = load_stream(src + rf_row_offset(g, g.layout, heads, b, n, nat) + c * 8);
    } else {
      val[p] = make_uint4(0, 0, 0, 0);
    }
  }

  __shared__ float red[kThreads * 8 > 128 * (D + 8) / 2 ? kThreads * 8 : 128 * (D + 8) / 2];

  if (kind == 2) {
    // V: stage the block in LDS, then write it transposed [D][128] with zero
    // columns past the block's length.
    if (a.mx) {
      // mxfp4: thread (channel d, part) quantises QPT consecutive key quarters
      // of channel d; codes of V^T two keys per byte ([D][64] bytes), the
      // quarter's E8M0 byte at row g, position DT (d % 32) + d / 32.
      constexpr int DT = D / 32;
      constexpr int QPT = 4 * D / kThreads;  // quarters per thread: 2 (D=128) or 1
      constexpr int TPD = 4 / QPT;           // threads per channel
      uint16_t* tile = reinterpret_cast<uint16_t*>(red);  // [128][D + 8]
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const int i = p * RPP + rsub;
        *reinterpret_cast<uint4*>(tile + i * (D + 8) + c * 8) = val[p];
      }
      __syncthreads();
      const int64_t blk = ((int64_t)b * g.N2 + n) * g.n_blocks + j;
      uint8_t* dst = reinterpret_cast<uint8_t*>(a.vpt) + blk * (int64_t)D * 64;
      uint8_t* sdst = reinterpret_cast<uint8_t*>(a.v_scale) + blk * 4 * D;
      const int d = tid / TPD, part = tid % TPD;
      uint32_t w[4 * QPT];
#pragma unroll
      for (int qq = 0; qq < QPT; ++qq) {
        const int gq = part * QPT + qq;
        float x[32];
        float amax = 0.0f;
#pragma unroll
        for (int r = 0; r < 32; ++r) {
          x[r] = __uint_as_float((uint32_t)tile[(32 * gq + r) * (D + 8) + d] << 16);
          amax = fmaxf(amax, fabsf(x[r]));
        }
        const int ex = rf_mx_scale_exp(amax);
#pragma unroll
        for (int r = 0; r < 32; ++r) x[r] = ldexpf(x[r], -ex);
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) w[4 * qq + k4] = rf_e2m1_pack8(x + 8 * k4);
        sdst[gq * D + DT * (d % 32) + d / 32] = (uint8_t)(ex + 127);
      }
#pragma unroll
      for (int qq = 0; qq < QPT; ++qq)
        store_stream(dst + d * 64 + (part * QPT + qq) * 16, w[4 * qq], w[4 * qq + 1],
                     w[4 * qq + 2], w[4 * qq + 3]);
      return;
    }
    if (a.v_scale) {
      // fp8: E4M3 codes of x / 2^e with the block's power-of-two scale 2^e
      // (exact scaling), same transposed layout in bytes.
      float amax = 0.0f;
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const uint32_t w[4] = {val[p].x, val[p].y, val[p].z, val[p].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          amax = fmaxf(amax, fmaxf(fabsf(bf_lo(w[e])), fabsf(bf_hi(w[e]))));
      }
      amax = block_max(amax, red);
      const int ex = pow2_scale_exp(amax);
      const float inv = ldexpf(1.0f, -ex);
      uint16_t* tile = reinterpret_cast<uint16_t*>(red);  // [128][D + 8]
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const int i = p * RPP + rsub;
        *reinterpret_cast<uint4*>(tile + i * (D + 8) + c * 8) = val[p];
      }
      __syncthreads();
      uint8_t* dst = reinterpret_cast<uint8_t*>(a.vpt) +
                     (((int64_t)b * g.N2 + n) * g.n_blocks + j) * (int64_t)D * 128;
#pragma unroll
      for (int m = 0; m < D / 32; ++m) {
        const int qd = tid + kThreads * m;
        const int d = qd / 8, cc = qd % 8;  // channel d, keys [16 cc, 16 cc + 16)
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float f[4];
#pragma unroll
          for (int bb = 0; bb < 4; ++bb)
            f[bb] = __uint_as_float((uint32_t)tile[(cc * 16 + 4 * e + bb) * (D + 8) + d] << 16) * inv;
          int x = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
          x = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], x, true);
          w[e] = (uint32_t)x;
        }
        store_stream(dst + d * 128 + cc * 16, w[0], w[1], w[2], w[3]);
      }
      if (tid == 0)
        static_cast<float*>(a.v_scale)[((int64_t)b * g.N2 + n) * g.n_blocks + j] = ldexpf(1.0f, ex);
      return;
    }
    uint16_t* tile = reinterpret_cast<uint16_t*>(red);  // [128][D + 8]
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int i = p * RPP + rsub;
      *reinterpret_cast<uint4*>(tile + i * (D + 8) + c * 8) = val[p];
    }
    __syncthreads();
    uint16_t* dst = a.vpt + (((int64_t)b * g.N2 + n) * g.n_blocks + j) * (int64_t)D * 128;
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
      const int qd = tid + kThreads * m;
      const int d = qd / 16, cc = qd % 16;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = tile[(cc * 8 + 2 * e) * (D + 8) + d];
        const uint32_t hi = tile[(cc * 8 + 2 * e + 1) * (D + 8) + d];
        w[e] = lo | (hi << 16);
      }
      store_stream(dst + d * 128 + cc * 8, w[0], w[1], w[2], w[3]);
    }
    return;
  }

  // Q or K: permuted bf16 copy.
  uint16_t* dstp = kind == 0 ? a.qp : a.kp;
  if (dstp) {
    const int64_t base = (((int64_t)b * heads + n) * g.S + row0) * D;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int i = p * RPP + rsub;
      if (i < len) store_stream(dstp + base + (int64_t)i * D + c * 8, val[p].x, val[p].y, val[p].z, val[p].w);
    }
  }

  // Block mean of a sparse block (fp32, fixed summation order).
  float* pool = kind == 0 ? a.q_pool : a.k_pool;
  const bool sparse_blk = j >= g.n_head && j < g.n_head + g.n_sparse;
  if (pool && sparse_blk) {
    float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const uint32_t w[4] = {val[p].x, val[p].y, val[p].z, val[p].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[2 * e] += bf_lo(w[e]);
        s[2 * e + 1] += bf_hi(w[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rsub * D + c * 8 + e] = s[e];
    __syncthreads();
    if (tid < D) {
      float t = 0.0f;
      for (int r = 0; r < RPP; ++r) t += red[r * D + tid];
      const int32_t js = j - g.n_head;
      pool[(((int64_t)b * heads + n) * g.n_sparse + js) * D + tid] = t * (1.0f / 128.0f);
    }
    __syncthreads();
  }

  uint8_t* q8 = kind == 0 ? a.q8 : a.k8;
  // mxfp4: E2M1 codes of each row's 32-channel blocks (4 adjacent threads hold
  // one block: 8 channels each) and one E8M0 byte per block.
  if (a.mx && q8) {
    constexpr int DT = D / 32;
    uint8_t* sc = reinterpret_cast<uint8_t*>(kind == 0 ? a.q_scale : a.k_scale);
    const int64_t rbase = ((int64_t)b * heads + n) * g.S + row0;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int i = p * RPP + rsub;
      const uint32_t w[4] = {val[p].x, val[p].y, val[p].z, val[p].w};
      float x[8];
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf_lo(w[e]);
        x[2 * e + 1] = bf_hi(w[e]);
        amax = fmaxf(amax, fmaxf(fabsf(x[2 * e]), fabsf(x[2 * e + 1])));
      }
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      amax = fmaxf(amax, __shfl_xor(amax, 2));
      const int ex = rf_mx_scale_exp(amax);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = ldexpf(x[e], -ex);
      const uint32_t codes = rf_e2m1_pack8(x);
      if (i < len) {
        *reinterpret_cast<uint32_t*>(q8 + (rbase + i) * (D / 2) + c * 4) = codes;
        if (c % 4 == 0) sc[(rbase + i) * DT + c / 4] = (uint8_t)(ex + 127);
      }
    }
    return;
  }
  // Mix precision: per-block E4M3 codes and scale.
  if (q8) {
    float amax = 0.0f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const uint32_t w[4] = {val[p].x, val[p].y, val[p].z, val[p].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        amax = fmaxf(amax, fmaxf(fabsf(bf_lo(w[e])), fabsf(bf_hi(w[e]))));
    }
    amax = block_max(amax, red);
    const float r = amax > 0.0f ? 448.0f / amax : 1.0f;
    const float sigma = amax > 0.0f ? amax / 448.0f : 1.0f;
    const int64_t base = (((int64_t)b * heads + n) * g.S + row0) * D;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int i = p * RPP + rsub;
      if (i < len) {
        const uint32_t w[4] = {val[p].x, val[p].y, val[p].z, val[p].w};
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(bf_lo(w[0]) * r, bf_hi(w[0]) * r, 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(bf_lo(w[1]) * r, bf_hi(w[1]) * r, lo, true);
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(bf_lo(w[2]) * r, bf_hi(w[2]) * r, 0, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(bf_lo(w[3]) * r, bf_hi(w[3]) * r, hi, true);
        store_stream(q8 + base + (int64_t)i * D + c * 8, (uint32_t)lo, (uint32_t)hi);
      }
    }
    float* sc = static_cast<float*>(kind == 0 ? a.q_scale : a.k_scale);
    if (tid == 0) sc[((int64_t)b * heads + n) * g.n_blocks + j] = sigma;
  }
}

struct UnpermuteArgs {
  RfGeom g;
  const uint16_t* out_p;
  uint16_t* out;
};

template <int D>
__global__ __launch_bounds__(kThreads) void unpermute_kernel(UnpermuteArgs a) {
  constexpr int C = D / 8;
  constexpr int RPP = kThreads / C;
  constexpr int PASSES = 128 / RPP;
  const RfGeom& g = a.g;
  const int tid = threadIdx.x;
  const int c = tid % C, rsub = tid / C;
  const int32_t j = blockIdx.x;
  const int32_t b = blockIdx.y / g.N1, n = blockIdx.y % g.N1;
  int64_t row0;
  int32_t len;
  rf_block_rows(g, j, &row0, &len);
  const uint16_t* src = a.out_p + (((int64_t)b * g.N1 + n) * g.S + row0) * D;
  uint4 val[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int i = p * RPP + rsub;
    if (i < len) val[p] = load_stream(src + (int64_t)i * D + c * 8);
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int i = p * RPP + rsub;
    if (i < len) {
      const int64_t nat = rf_natural_row(g, row0 + i);
      store_stream(a.out + rf_row_offset(g, g.layout, g.N1, b, n, nat) + c * 8, val[p].x, val[p].y,
                   val[p].z, val[p].w);
    }
  }
}

}  // namespace

rf_status rf_launch_permute(const RfGeom& g, int32_t precision, const void* q, const void* k,
                            const void* v, void* qp, void* kp, void* vpt, float* q_pool,
                            float* k_pool, uint8_t* q8, uint8_t* k8, void* q_scale,
                            void* k_scale, void* v_scale, void* stream) {
  PermuteArgs a;
  a.mx = precision == RF_PREC_MXFP4;
  a.g = g;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.qp = static_cast<uint16_t*>(qp);
  a.kp = static_cast<uint16_t*>(kp);
  a.vpt = static_cast<uint16_t*>(vpt);
  a.q_pool = q_pool;
  a.k_pool = k_pool;
  a.q8 = q8;
  a.k8 = k8;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  const dim3 grid(g.n_blocks, g.B * (g.N1 + 2 * g.N2));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.D == 128)
    hipLaunchKernelGGL(permute_kernel<128>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(permute_kernel<64>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? RF_OK : RF_ERR_HIP;
}

rf_status rf_launch_unpermute(const RfGeom& g, const void* out_p, void* out, void* stream) {
  UnpermuteArgs a;
  a.g = g;
  a.out_p = static_cast<const uint16_t*>(out_p);
  a.out = static_cast<uint16_t*>(out);
  const dim3 grid(g.n_blocks, g.B * g.N1);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.D == 128)
    hipLaunchKernelGGL(unpermute_kernel<128>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(unpermute_kernel<64>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? RF_OK : RF_ERR_HIP;
}
