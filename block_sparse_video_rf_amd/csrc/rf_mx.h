// E2M1 packing shared by the device code that quantises (the permute kernel:
// Q, K, V) and the attention kernel (P). The block exponent rule,
// rf_mx_scale_exp, is in rf_internal.h (host and device).
#ifndef RF_MX_H_
#define RF_MX_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rf_internal.h"

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
