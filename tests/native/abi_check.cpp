// The whole path driven through the C ABI of librf.so with plain HIP runtime
// calls: no Python, no torch. Checks properties that hold at any size:
//   1. rf_dense_attn equals rf_sparse_attn given every block, bit for bit;
//   2. with V constant, the output of the whole path (permute, pool/select,
//      sparse attention, unpermute) is that constant (attention is a weighted
//      average of V rows), within one bf16 ulp;
//   3. argument errors come back as status codes and enqueue nothing.
// Usage: abi_check [bf16|mix|fp8]. Prints "abi_check ok" and exits 0 on success.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "rf.h"

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 2;                                                                \
    }                                                                          \
  } while (0)
#define RF_OK_(x)                                                              \
  do {                                                                         \
    rf_status s_ = (x);                                                        \
    if (s_ != RF_OK) {                                                         \
      std::fprintf(stderr, "%s failed: %s\n", #x, rf_status_str(s_));          \
      return 3;                                                                \
    }                                                                          \
  } while (0)

static uint16_t to_bf16(float f) {  // round to nearest even
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

template <typename T>
static T* dev_alloc(size_t n, std::vector<void*>& owned) {
  void* p = nullptr;
  if (n == 0) n = 1;
  if (hipMalloc(&p, n * sizeof(T)) != hipSuccess) {
    std::fprintf(stderr, "hipMalloc of %zu bytes failed\n", n * sizeof(T));
    std::exit(2);
  }
  owned.push_back(p);
  return static_cast<T*>(p);
}

int main(int argc, char** argv) {
  const char* prec = argc > 1 ? argv[1] : "bf16";
  rf_desc d;
  std::memset(&d, 0, sizeof(d));
  d.layout = RF_LAYOUT_BNSD;
  d.dtype = RF_DTYPE_BF16;
  d.batch = 1;
  d.heads_q = 4;
  d.heads_kv = 2;  // grouped-query attention
  d.head_dim = 128;
  d.prefix_len = 200;  // not a multiple of 128
  d.grid_t = 10;
  d.grid_h = 17;
  d.grid_w = 34;  // unaligned height and width, an unpaired last frame
  d.first_frame_rows = (int64_t)d.grid_h * d.grid_w;
  d.seq_len = d.prefix_len + (int64_t)d.grid_t * d.grid_h * d.grid_w;
  d.block_shape[0] = d.block_shape[1] = 128;
  d.precision = !std::strcmp(prec, "mix") ? RF_PREC_MIX
                : !std::strcmp(prec, "fp8") ? RF_PREC_FP8 : RF_PREC_BF16;
  d.sparsity = 0.8;
  d.scale = 1.0f / std::sqrt(128.0f);
  d.min_sparse_blocks = 1;
  rf_plan_info pi;
  RF_OK_(rf_plan(&d, &pi));
  const bool qk8 = d.precision != RF_PREC_BF16, v8 = d.precision == RF_PREC_FP8;
  const int64_t nq = pi.qp_elems, nk = pi.kp_elems;
  std::printf("abi_check %s: S=%lld blocks=%d sparse=%d topk=%d\n", prec, (long long)d.seq_len,
              pi.n_blocks, pi.n_sparse, pi.topk);

  // Inputs: a fixed pseudo-random Q and K in [-2, 2); V random or constant.
  std::vector<uint16_t> hq(nq), hk(nk), hv(nk), hv1(nk, to_bf16(0.75f));
  uint32_t st = 12345u;
  auto rnd = [&]() { st = st * 1664525u + 1013904223u; return ((st >> 8) & 0xffff) / 16384.0f - 2.0f; };
  for (auto& x : hq) x = to_bf16(rnd());
  for (auto& x : hk) x = to_bf16(rnd());
  for (auto& x : hv) x = to_bf16(rnd());

  std::vector<void*> owned;
  auto* q = dev_alloc<uint16_t>(nq, owned);
  auto* k = dev_alloc<uint16_t>(nk, owned);
  auto* v = dev_alloc<uint16_t>(nk, owned);
  auto* qp = qk8 ? nullptr : dev_alloc<uint16_t>(nq, owned);
  auto* kp = qk8 ? nullptr : dev_alloc<uint16_t>(pi.kp_elems, owned);  // natural size
  auto* vpt = dev_alloc<uint16_t>(pi.vpt_elems, owned);  // E4M3 codes need half of it
  auto* q_pool = dev_alloc<float>(pi.q_pool_elems, owned);
  auto* k_pool = dev_alloc<float>(pi.k_pool_elems, owned);
  auto* q8 = qk8 ? dev_alloc<uint8_t>(nq, owned) : nullptr;
  auto* k8 = qk8 ? dev_alloc<uint8_t>(pi.k8_bytes, owned) : nullptr;
  auto* q_scale = qk8 ? dev_alloc<float>(pi.q_scale_elems, owned) : nullptr;
  auto* k_scale = qk8 ? dev_alloc<float>(pi.k_scale_elems, owned) : nullptr;
  auto* v_scale = v8 ? dev_alloc<float>(pi.v_scale_elems, owned) : nullptr;
  const int32_t max_kv = pi.max_kv_blocks;
  const size_t nidx = (size_t)pi.select_rows * d.heads_q * max_kv;
  const size_t nnum = (size_t)pi.select_rows * d.heads_q;
  auto* sel_idx = dev_alloc<int32_t>(nidx, owned);
  auto* sel_num = dev_alloc<int32_t>(nnum, owned);
  auto* ws = dev_alloc<uint8_t>(pi.ws_select_bytes, owned);
  auto* out_p = dev_alloc<uint16_t>(nq, owned);
  auto* out_p2 = dev_alloc<uint16_t>(nq, owned);
  auto* out = dev_alloc<uint16_t>(nq, owned);
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  HIP_OK(hipMemcpy(q, hq.data(), nq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk.data(), nk * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv.data(), nk * 2, hipMemcpyHostToDevice));

  // 1. Dense entry point against the sparse one given every block.
  RF_OK_(rf_permute(&d, q, k, v, qp, kp, vpt, nullptr, nullptr, q8, k8, q_scale, k_scale, v_scale, s));
  std::vector<int32_t> all_idx(nidx), all_num(nnum, pi.n_blocks);
  for (size_t r = 0; r < nnum; ++r)
    for (int32_t j = 0; j < max_kv; ++j) all_idx[r * max_kv + j] = j < pi.n_blocks ? j : -1;
  HIP_OK(hipMemcpy(sel_idx, all_idx.data(), nidx * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(sel_num, all_num.data(), nnum * 4, hipMemcpyHostToDevice));
  RF_OK_(rf_sparse_attn(&d, qp, kp, vpt, q8, k8, q_scale, k_scale, v_scale, sel_idx, sel_num,
                        max_kv, out_p, s));
  RF_OK_(rf_dense_attn(&d, qp, kp, vpt, q8, k8, q_scale, k_scale, v_scale, out_p2, s));
  HIP_OK(hipStreamSynchronize(s));
  std::vector<uint16_t> a(nq), b(nq);
  HIP_OK(hipMemcpy(a.data(), out_p, nq * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(b.data(), out_p2, nq * 2, hipMemcpyDeviceToHost));
  if (std::memcmp(a.data(), b.data(), nq * 2) != 0) {
    std::fprintf(stderr, "dense path differs from the sparse kernel with every block\n");
    return 1;
  }

  // 2. Constant V through the whole path.
  HIP_OK(hipMemcpy(v, hv1.data(), nk * 2, hipMemcpyHostToDevice));
  RF_OK_(rf_permute(&d, q, k, v, qp, kp, vpt, q_pool, k_pool, q8, k8, q_scale, k_scale, v_scale, s));
  RF_OK_(rf_pool_select(&d, qp, kp, q_pool, k_pool, sel_idx, sel_num, max_kv, ws,
                        pi.ws_select_bytes, s));
  RF_OK_(rf_sparse_attn(&d, qp, kp, vpt, q8, k8, q_scale, k_scale, v_scale, sel_idx, sel_num,
                        max_kv, out_p, s));
  RF_OK_(rf_unpermute(&d, out_p, out, s));
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(a.data(), out, nq * 2, hipMemcpyDeviceToHost));
  double worst = 0.0;
  for (int64_t i = 0; i < nq; ++i) worst = std::fmax(worst, std::fabs(from_bf16(a[i]) - 0.75));
  if (!(worst <= 1.0 / 256.0)) {  // one bf16 ulp at 0.75
    std::fprintf(stderr, "constant V: worst deviation %g\n", worst);
    return 1;
  }

  // 3. Errors: a NULL output, an aliased output, a bad descriptor.
  if (rf_unpermute(&d, out_p, nullptr, s) != RF_ERR_NULL) return 1;
  if (rf_unpermute(&d, out_p, out_p, s) != RF_ERR_ALIAS) return 1;
  rf_desc bad = d;
  bad.heads_kv = 3;
  if (rf_plan(&bad, &pi) != RF_ERR_GQA) return 1;

  HIP_OK(hipStreamDestroy(s));
  for (void* p : owned) HIP_OK(hipFree(p));
  std::printf("abi_check ok (%s): dense == sparse with every block; constant V within %g\n", prec,
              worst);
  return 0;
}
