// Achievable LDS bandwidth and vector-ALU issue costs on this GPU, in shader
// clock cycles (s_memtime), to read the attention kernel's counters against.
//
// LDS: one workgroup of 8 waves per CU (96 KiB of LDS keeps it alone on its
// CU); every lane moves 16-byte chunks of a 64 KiB buffer, consecutive lanes
// at consecutive chunks (no bank conflicts), 8 accesses in flight per wave.
//   reads:  ds_read_b128 only;  writes: ds_write_b128 only.
// VALU: one workgroup of 8 waves per CU (two per SIMD); every wave runs 16
// independent register chains of one instruction (v_exp_f32, or v_fma_f32 as
// the full-rate reference), so the figure is the issue cost of one wave64
// instruction on its SIMD.
// Prints one JSON object.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLdsIters = 4096;   // 16-byte accesses per lane
constexpr int kValuIters = 512;   // rounds of 16 instructions per wave

template <int WRITE>
__global__ __launch_bounds__(512) void lds_loop(uint64_t* cycles, uint32_t* sink, int salt) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[98304];
  const int tid = threadIdx.x;
  for (int i = tid; i < 98304 / 16; i += 512)
    reinterpret_cast<u32x4*>(buf)[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  const int wave = tid / 64, lane = tid % 64;
  u32x4 acc = {0, 0, 0, 0};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < kLdsIters; it += 8) {
    asm volatile("" ::: "memory");  // keeps every access inside the loop
    if (WRITE) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int off = (((it + k) * 8 + wave) * 1024 + lane * 16) & 32767;
        *reinterpret_cast<u32x4*>(buf + 65536 + off) = u32x4{(uint32_t)(it + k), 0u, 0u, 0u};
      }
    } else {
      u32x4 r[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int off = (((it + k) * 8 + wave + salt) * 1024 + lane * 16) & 65535;
        r[k] = *reinterpret_cast<const u32x4*>(buf + off);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) acc += r[k];
    }
  }
  __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (tid == 0) cycles[blockIdx.x] = t1 - t0;
  sink[blockIdx.x * 512 + tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

#define RF_CHAIN16(OP)                                                                   \
  asm volatile(OP " %0, %0\n\t" OP " %1, %1\n\t" OP " %2, %2\n\t" OP " %3, %3\n\t"      \
               OP " %4, %4\n\t" OP " %5, %5\n\t" OP " %6, %6\n\t" OP " %7, %7"           \
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), \
                 "+v"(x[6]), "+v"(x[7]));                                                \
  asm volatile(OP " %0, %0\n\t" OP " %1, %1\n\t" OP " %2, %2\n\t" OP " %3, %3\n\t"      \
               OP " %4, %4\n\t" OP " %5, %5\n\t" OP " %6, %6\n\t" OP " %7, %7"           \
               : "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]),          \
                 "+v"(x[13]), "+v"(x[14]), "+v"(x[15]))

#define RF_FMA16                                                                         \
  asm volatile("v_fma_f32 %0, %0, %8, %8\n\tv_fma_f32 %1, %1, %8, %8\n\t"                \
               "v_fma_f32 %2, %2, %8, %8\n\tv_fma_f32 %3, %3, %8, %8\n\t"                \
               "v_fma_f32 %4, %4, %8, %8\n\tv_fma_f32 %5, %5, %8, %8\n\t"                \
               "v_fma_f32 %6, %6, %8, %8\n\tv_fma_f32 %7, %7, %8, %8"                    \
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), \
                 "+v"(x[6]), "+v"(x[7])                                                  \
               : "v"(h));                                                                \
  asm volatile("v_fma_f32 %0, %0, %8, %8\n\tv_fma_f32 %1, %1, %8, %8\n\t"                \
               "v_fma_f32 %2, %2, %8, %8\n\tv_fma_f32 %3, %3, %8, %8\n\t"                \
               "v_fma_f32 %4, %4, %8, %8\n\tv_fma_f32 %5, %5, %8, %8\n\t"                \
               "v_fma_f32 %6, %6, %8, %8\n\tv_fma_f32 %7, %7, %8, %8"                    \
               : "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]),          \
                 "+v"(x[13]), "+v"(x[14]), "+v"(x[15])                                   \
               : "v"(h))

template <int EXP>
__global__ __launch_bounds__(512) void valu_loop(uint64_t* cycles, float* sink, float seed) {
  float x[16];
  for (int i = 0; i < 16; ++i) x[i] = seed * (float)(i + 1) * 1e-3f;
  const float h = 0.5f;
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < kValuIters; ++it) {
    if (EXP) {
      RF_CHAIN16("v_exp_f32");
    } else {
      RF_FMA16;
    }
  }
  __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) cycles[blockIdx.x] = t1 - t0;
  float s = 0.0f;
  for (int i = 0; i < 16; ++i) s += x[i];
  sink[blockIdx.x * 512 + threadIdx.x] = s;
}

int main(int argc, char** argv) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 2;
  const int grid = cus;  // one workgroup per CU
  const int salt = argc > 99 ? 1 : 0;  // 0 at run time, opaque to the compiler
  uint64_t* cyc = nullptr;
  uint32_t* sink = nullptr;
  if (hipMalloc(&cyc, (size_t)grid * sizeof(uint64_t)) != hipSuccess ||
      hipMalloc(&sink, (size_t)grid * 512 * sizeof(uint32_t)) != hipSuccess)
    return 2;
  uint64_t* h = new uint64_t[grid];
  auto mean_cycles = [&]() -> double {
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(h, cyc, (size_t)grid * sizeof(uint64_t), hipMemcpyDeviceToHost) != hipSuccess)
      return -1.0;
    double m = 0.0;
    for (int i = 0; i < grid; ++i) m += (double)h[i] / grid;
    return m;
  };
  double res[4];
  for (int kind = 0; kind < 4; ++kind) {
    double best = 1e300;
    for (int rep = 0; rep < 3; ++rep) {
      if (kind == 0) hipLaunchKernelGGL(lds_loop<0>, dim3(grid), dim3(512), 0, 0, cyc, sink, salt);
      if (kind == 1) hipLaunchKernelGGL(lds_loop<1>, dim3(grid), dim3(512), 0, 0, cyc, sink, salt);
      if (kind == 2)
        hipLaunchKernelGGL(valu_loop<1>, dim3(grid), dim3(512), 0, 0, cyc,
                           reinterpret_cast<float*>(sink), 1.0f);
      if (kind == 3)
        hipLaunchKernelGGL(valu_loop<0>, dim3(grid), dim3(512), 0, 0, cyc,
                           reinterpret_cast<float*>(sink), 1.0f);
      if (hipGetLastError() != hipSuccess) return 2;
      const double m = mean_cycles();
      if (m <= 0.0) return 2;
      if (m < best) best = m;
    }
    res[kind] = best;
  }
  const double lds_bytes = 512.0 * 16 * kLdsIters;      // per workgroup (= per CU)
  const double valu_insts = 2.0 * 16 * kValuIters;      // per SIMD (two waves)
  std::printf("{\"cus\": %d, \"lds_read_B_per_clk_per_cu\": %.1f, "
              "\"lds_write_B_per_clk_per_cu\": %.1f, \"v_exp_f32_cycles\": %.2f, "
              "\"v_fma_f32_cycles\": %.2f}\n",
              cus, lds_bytes / res[0], lds_bytes / res[1], res[2] / valu_insts,
              res[3] / valu_insts);
  delete[] h;
  hipFree(cyc);
  hipFree(sink);
  return 0;
}
