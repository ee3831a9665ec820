// MXFP4 scale rule shared by the device code that quantises (the permute
// kernel: Q, K, V) and the attention kernel (P).
//
// "MXAttention: Data-Free Optimal Scaling and Pre-Normalization Quantization
// for MXFP4 Attention", abstract: power-of-two (E8M0) block scales with the
// boundary Qmax = 7.25. The block exponent is the smallest e with
// amax <= 7.25 * 2^e, clamped to the E8M0 range [-127, 127]. With
// amax = m * 2^E, m in [1, 2), and 7.25 = 1.8125 * 2^2: e = E - 2 if
// m <= 1.8125, else E - 1 -- exact, from the bits. Zero and subnormal maxima
// (below 2^-126 < 7.25 * 2^-127) give -127.
#ifndef RF_MX_H_
#define RF_MX_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

__device__ __forceinline__ int rf_mx_scale_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int eb = (int)(u >> 23);
  if (eb == 0) return -127;
  const int e = eb - 129 + ((u & 0x7fffffu) > 0x680000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// E2M1 codes (nearest even, saturating at +-6) of y[0..7], two per byte with
// y[2i] in the low nibble of byte i: one conversion instruction per byte.
__device__ __forceinline__ uint32_t rf_e2m1_pack8(const float* y) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}

#endif  // RF_MX_H_
