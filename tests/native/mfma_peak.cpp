// Achievable matrix-core throughput on this GPU: every wave of a full grid
// issues independent chains of one MFMA from registers (no memory traffic
// but one store per lane at the end). Prints one JSON object with the bf16
// (v_mfma_f32_32x32x16_bf16) and fp8 (v_mfma_scale_f32_32x32x64_f8f6f4)
// rates in TFLOP/s.
#include <hip/hip_runtime.h>

#include <cstdio>

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

constexpr int kIters = 4096;  // products per chain
constexpr int kChains = 4;

__global__ __launch_bounds__(512, 1) void bf16_loop(float* out, int seed) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((threadIdx.x + i + seed) & 3);
    b[i] = (__bf16)(float)((threadIdx.x * 3 + i) & 3);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < kIters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * 512 + threadIdx.x] = s;
}

__global__ __launch_bounds__(512, 1) void fp8_loop(float* out, int seed) {
  i32x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 ^ ((threadIdx.x + i + seed) & 1);
    b[i] = 0x30303030;
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < kIters; ++it) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 0, 0, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 0, 0, 0, 127, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 0, 0, 0, 127, 0, 127);
  }
  float s = 0.0f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * 512 + threadIdx.x] = s;
}

int main() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 2;
  const int grid = cus * 4;  // several workgroups of 8 waves per CU, in turn
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)grid * 512 * sizeof(float)) != hipSuccess) return 2;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 2;
  const double waves = (double)grid * 8;
  double tf[2];
  for (int kind = 0; kind < 2; ++kind) {
    float best = 1e30f;
    for (int rep = 0; rep < 3; ++rep) {
      if (hipEventRecord(e0, 0) != hipSuccess) return 2;
      if (kind == 0)
        hipLaunchKernelGGL(bf16_loop, dim3(grid), dim3(512), 0, 0, out, rep);
      else
        hipLaunchKernelGGL(fp8_loop, dim3(grid), dim3(512), 0, 0, out, rep);
      if (hipGetLastError() != hipSuccess || hipEventRecord(e1, 0) != hipSuccess ||
          hipEventSynchronize(e1) != hipSuccess)
        return 2;
      float ms = 0.0f;
      if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return 2;
      if (ms < best) best = ms;
    }
    // flops per product: 2 * 32 * 32 * 16 (bf16) or 2 * 32 * 32 * 64 (fp8)
    const double per = kind == 0 ? 32768.0 : 131072.0;
    tf[kind] = waves * kChains * kIters * per / (best * 1e-3) / 1e12;
  }
  std::printf("{\"cus\": %d, \"mfma_bf16_tflops\": %.1f, \"mfma_fp8_tflops\": %.1f}\n", cus, tf[0],
              tf[1]);
  hipFree(out);
  return 0;
}
