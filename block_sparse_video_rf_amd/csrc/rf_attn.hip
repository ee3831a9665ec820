// Block-sparse attention: exact softmax(scale * Q K^T) V over the key blocks
// listed in selectIdx ("aclnnRainFusionAttention", Formula; 128 x 128 blocks).
//
// One workgroup of 8 waves per (batch, query block, query head). Wave w owns
// query rows [32 rg, 32 rg + 32) of the block (rg = w % 4) and one half of the
// keys of every listed block (kh = 1 - w / 4). The workgroup walks its list of key
// blocks, staging K (row-major, [128][D]) and V (already block-transposed by
// the permute kernel, [D][128]) in LDS, and each wave computes
//
//   S^T = K Q^T  with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS,
//                B = the wave's Q rows, held in registers for the whole walk)
//   online softmax in fp32, exp2 with the scale folded in
//   O^T += V^T P^T  with the same MFMA (A = V^T rows from LDS, B = P in bf16)
//
// Computing the transposed products makes every lane own one query row
// (column l % 32 of the 32x32 accumulator tiles), so the row maximum, the
// running sum and the rescale of O are lane-local except for one exchange
// with the partner lane l ^ 32 for the maximum (when one is needed: bf16 and
// mix take the exponentials against the running reference and compute a
// maximum only when a block's sums say the reference must rise).
//
// K rows are fed to the A operand in a permuted order (kappa(), which swaps
// bits 2 and 3 of the tile row) so that the 16 accumulator values of a lane
// in a tile cover key rows 16*(v/8) + 8*(l/32) + v%8: each group of 8 is
// contiguous, which is exactly the 8-value k-slice the PV product wants from
// the B operand, and the matching V^T slice is one contiguous 16-byte LDS
// read.
//
// The two waves on each SIMD (same rg) run half an iteration apart, so that
// one issues matrix products while the other runs the softmax: the schedule
// is described at the kernel.
//
// The mix precision replaces the QK^T operands by fp8 E4M3 codes
// (v_mfma_scale_f32_32x32x64_f8f6f4, unit block scales) and folds
// scale * q_scale * k_scale of the block pair into the exponent multiplier.
// The fp8 precision also runs O^T on E4M3 codes: V^T codes with the block's
// power-of-two scale as the product's E8M0 operand scale, and P quantised to
// E4M3 with the row's power-of-two block scale (the smallest 2^m with
// 2^(max t) <= 448 * 2^m, raised as blocks arrive, so the largest P lies in
// (224, 448]); an extra product of an all-ones operand with P^T gives the row
// sums of the rounded P. The mxfp4 precision runs both
// products on E2M1 codes with one E8M0 scale per 32 values of each operand
// lane (the MX block of the hardware: a lane's 32 contraction values): Q and
// K scales per 32 channels, V^T scales per 32 keys, and P quantised per lane
// (its 32 keys of one query row) with the scale rule of rf_mx.h, against the
// same integer reference as fp8. With no lists (the dense path) every block is
// visited in order.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "rf_internal.h"
#include "rf_mx.h"

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

// The scaled 32x32x64 product with E2M1 operands in 4 registers each: the
// v4i32 overload of the LLVM intrinsic (the clang builtin only takes the
// 8-register operands of fp8). cbsz = blgp = 4 selects E2M1; opsel picks the
// byte of each lane's 32-bit scale word that holds its E8M0 scale.
__device__ f32x16_t rf_mfma_scale_fp4(i32x4 a, i32x4 b, f32x16_t c, int cbsz, int blgp,
                                      int opsel_a, int scale_a, int opsel_b, int scale_b)
    __asm("llvm.amdgcn.mfma.scale.f32.32x32x64.f8f6f4.v4i32.v4i32");

namespace {

constexpr int kThreads8 = 512;  // attention workgroup: 8 waves
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct AttnArgs {
  RfGeom g;
  float scale_log2;  // scale * log2(e)
  const uint16_t* qp;
  const uint16_t* kp;
  const uint16_t* vpt;
  const uint8_t* q8;
  const uint8_t* k8;
  const void* q_scale;  // fp32 per block (mix, fp8); E8M0 bytes (mxfp4)
  const void* k_scale;
  const void* v_scale;
  const int32_t* select_idx;
  const int32_t* select_num;
  int32_t max_kv;
  uint16_t* out_p;
};

__device__ __forceinline__ int kappa(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Key row order for fp8 O^T products: A-operand row i of key tile t holds key
// 16 t + kappa8(i) of the wave's 64, kappa8(i) = (i & 3) + 4 (i >> 3) +
// 32 ((i >> 2) & 1), which puts keys 32 (l / 32) + [0, 32) in lane l's two
// accumulator tiles (tile t, value v = key 32 (l / 32) + 16 t + v): exactly the
// 32-byte k-slice of the fp8 B operand, in order. Reading rows kappa8(i)
// directly would put rows r and r + 32 in one 16-lane read (the same banks for
// any 16-byte-aligned stride), so the K tile is stored in that order instead:
// key r of the 128-row block goes to LDS row kslot8(r), and lane i of key tile
// t reads row 64 kh + 32 t + i.
__device__ __forceinline__ int kslot8(int r) {
  return (r & 64) | (((r >> 4) & 1) << 5) | (((r >> 2) & 3) << 3) | (((r >> 5) & 1) << 2) |
         (r & 3);
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

// Scalar view of one float array (k_scale): uniform reads become s_load.
typedef const float __attribute__((address_space(4)))* scale_ptr;

// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left at their
// maxima (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVmcnt0 = 0x0F70;

// Raw buffer descriptor over [base, base + bytes). The hardware compares the
// whole offset of a load (SGPR offset + VGPR offset + immediate) with `bytes`
// and returns zeros past it (measured on MI355X), so the K tile of a short
// block at the end of the sequence reads zeros past the sequence and nothing
// outside the buffer is touched. (Third dword: the raw 32-bit data format used
// for plain byte-addressed buffers on gfx9.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Workgroup barrier that waits only for this wave's LDS operations: tile
// prefetches from global memory stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier after which this wave's LDS stores are visible, while its
// last N LDS operations (reads) may still be in flight: LDS operations of a
// wave complete in issue order, so at most N outstanding means every earlier
// one (the stores) is done. Scalar loads count too, which only makes the wait
// stricter. The caller keeps those N reads last (a scheduling fence before
// them).
template <int N>
__device__ __forceinline__ void lds_barrier_keep() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Maxima without the NaN canonicalisation fmaxf needs (no NaN reaches them:
// masked scores are -inf).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// Maximum of a lane's value and that of lane l ^ 32 (v_permlane32_swap hands
// every lane its own value and its partner's).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max3f(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}

// Operand modes: bf16 products; mix (fp8 E4M3 S^T = K Q^T, bf16 O^T); fp8
// (both products on E4M3 codes); mxfp4 (both products on E2M1 codes).
template <int PREC>
struct Prec {
  static constexpr bool QK8 = PREC != RF_PREC_BF16;  // S^T on quantised codes
  static constexpr bool F4 = PREC == RF_PREC_MXFP4;  // E2M1 operands, per-lane E8M0 scales
  static constexpr bool VQ = PREC == RF_PREC_FP8 || F4;  // O^T on codes, P quantised
};

// Operand schedule of one MFMA interval: the S^T products of this block
// (A = K rows from LDS) followed by the O^T products of the previous block
// (A = V^T rows from LDS). Every LDS read is one 16-byte fragment per lane;
// an fp8 product takes two.
template <int D, int PREC>
struct MfmaPlan {
  static constexpr bool QK8 = Prec<PREC>::QK8, VQ = Prec<PREC>::VQ, F4 = Prec<PREC>::F4;
  static constexpr int DT = D / 32;
  static constexpr int QK_STEPS = QK8 ? D / 64 : D / 16;
  static constexpr int S_RPM = QK8 && !F4 ? 2 : 1;   // reads per S^T product
  static constexpr int NS_MFMA = 2 * QK_STEPS;       // S^T products (2 key tiles)
  static constexpr int NS_READ = NS_MFMA * S_RPM;
  // O^T products: DT channel tiles x the wave's 64 keys in k-steps of 16
  // (bf16) or one k-step of 64 (fp8, mxfp4).
  static constexpr int NPV = VQ ? DT : 4 * DT;
  static constexpr int PV_RPM = VQ && !F4 ? 2 : 1;   // reads per O^T product
  static constexpr int NREAD = NS_READ + NPV * PV_RPM;
  // fp8, mxfp4: one more product, of an all-ones A operand with P^T,
  // accumulates the row sums of the rounded P (no LDS reads).
  static constexpr int NSUM = VQ ? 1 : 0;
  static constexpr int NMFMA = NS_MFMA + NPV + NSUM;
  static constexpr int NR = 8;                       // fragments in flight
  static constexpr int NPRE = NR < NS_READ ? NR : NS_READ;  // K reads issued before the barrier
  static constexpr int rend(int m) {
    return m < NS_MFMA ? (m + 1) * S_RPM
                       : (m < NS_MFMA + NPV ? NS_READ + (m - NS_MFMA + 1) * PV_RPM : NREAD);
  }
};

// Ring of fragments in named registers (an array could be placed in scratch).
struct FragRing {
  uint4 r0, r1, r2, r3, r4, r5, r6, r7;
};
template <int I>
__device__ __forceinline__ uint4& ring_slot(FragRing& f) {
  static_assert(I >= 0 && I < 8, "ring slot");
  if constexpr (I == 0) return f.r0;
  else if constexpr (I == 1) return f.r1;
  else if constexpr (I == 2) return f.r2;
  else if constexpr (I == 3) return f.r3;
  else if constexpr (I == 4) return f.r4;
  else if constexpr (I == 5) return f.r5;
  else if constexpr (I == 6) return f.r6;
  else return f.r7;
}

template <int D, int PREC>
struct MfmaCtx {
  using P = MfmaPlan<D, PREC>;
  const uint8_t* kbase;  // this lane's first K fragment in the current K buffer
  const uint8_t* vbase;  // this lane's first V^T fragment in the previous block's buffer
  FragRing ring;
  f32x16 s[2];
  f32x16 o[P::DT];
  bf16x8 qf[P::QK8 ? 1 : P::QK_STEPS];
  i32x8 qf8[P::QK8 && !P::F4 ? P::QK_STEPS : 1];
  i32x4 qf4[P::F4 ? P::QK_STEPS : 1];  // Q fragment (E2M1 codes), mxfp4
  bf16x8 pf16[2][2];              // P^T operands, bf16 O^T products
  i32x8 pf8;                      // P^T operand (E4M3 codes), fp8 O^T products
  i32x4 pf4;                      // P^T operand (E2M1 codes), mxfp4 O^T products
  int vexp;                       // E8M0 scale of the previous block's V (fp8)
  // mxfp4 E8M0 scale words (byte = scale of one operand lane's 32 values):
  // Q (byte 2 st: k-step st), K per key tile (likewise), V^T of the previous
  // block (byte e: channel tile e).
  int qsc, ksc[2], vsc;
  // fp8, mxfp4: E8M0 scale of the P^T operand (byte 0): 2^(m_run - m_ref),
  // times the lane's MX scale in mxfp4.
  int psc;
  f32x16 osum;                    // fp8, mxfp4: every value is the running row sum of P
};

// Bytes per row of a K tile and of a V^T tile in global memory, and their
// padded LDS strides (the padding spreads a wave's 16-byte reads over all
// banks).
template <int D, int PREC>
struct TileGeom {
  static constexpr bool F4 = Prec<PREC>::F4;
  static constexpr int KROW = F4 ? D / 2 : (Prec<PREC>::QK8 ? D : 2 * D);
  static constexpr int VROW = F4 ? 64 : (Prec<PREC>::VQ ? 128 : 256);
  static constexpr int KSTR = KROW + 16;
  static constexpr int VSTR = VROW + 16;
  // mxfp4: the E8M0 bytes that follow a tile in LDS: D/32 per K row (in the
  // rows' LDS order), 4 x D per V^T tile (the layout rf_permute writes); both
  // 4 D bytes.
  static constexpr int KSC = F4 ? 128 * (D / 32) : 0;
  static constexpr int VSC = F4 ? 4 * D : 0;
};

// LDS byte offset of read R relative to its base (compile-time).
template <int D, int PREC, int R>
__device__ __forceinline__ const uint8_t* read_addr(const MfmaCtx<D, PREC>& c) {
  using P = MfmaPlan<D, PREC>;
  using TG = TileGeom<D, PREC>;
  if constexpr (R < P::NS_READ) {
    // S^T product sm: key tile t (LDS rows 32 t + [0, 32)), channel k-step st.
    constexpr int sm = R / P::S_RPM, half = R % P::S_RPM, st = sm / 2, t = sm % 2;
    return c.kbase + 32 * t * TG::KSTR + (P::QK8 && !P::F4 ? 64 * st + 16 * half : 32 * st);
  } else if constexpr (P::VQ) {
    // O^T product e (channel tile): the lane's 32 keys of V^T row 32 e + li
    // (32 bytes of E4M3, 16 of E2M1).
    constexpr int pr = R - P::NS_READ, e = pr / P::PV_RPM, half = pr % P::PV_RPM;
    return c.vbase + 32 * e * TG::VSTR + 16 * half;
  } else {
    constexpr int pm = R - P::NS_READ, tu = pm / P::DT, e = pm % P::DT;
    return c.vbase + 32 * e * TG::VSTR + 2 * (32 * (tu / 2) + 16 * (tu % 2));
  }
}

template <int D, int PREC, int R, int END>
__device__ __forceinline__ void issue_reads(MfmaCtx<D, PREC>& c) {
  using P = MfmaPlan<D, PREC>;
  if constexpr (R < END && R < P::NREAD) {
    ring_slot<R % P::NR>(c.ring) = *reinterpret_cast<const uint4*>(read_addr<D, PREC, R>(c));
    issue_reads<D, PREC, R + 1, END>(c);
  }
}

// Keeps every product of an MFMA interval inside it. The scaled fp8 product
// intrinsic can be sunk by the compiler's IR passes (sched_barrier only binds
// the machine scheduler) into the next interval, next to the first use of its
// result, which would serialise it with the softmax. An empty asm statement
// that takes the accumulators as inputs must follow their products. (The host
// pass of the compiler parses device code too and has no VGPR tuples: the
// statements exist for the device pass only.)
__device__ __forceinline__ void pin_acc(const f32x16& x) {
#if __HIP_DEVICE_COMPILE__
  asm volatile("" ::"v"(x));
#else
  (void)x;
#endif
}
template <int D, int PREC>
__device__ __forceinline__ void pin_products(MfmaCtx<D, PREC>& c) {
  pin_acc(c.s[0]);
  pin_acc(c.s[1]);
#pragma unroll
  for (int e = 0; e < MfmaPlan<D, PREC>::DT; ++e) pin_acc(c.o[e]);
  if constexpr (Prec<PREC>::VQ) pin_acc(c.osum);
}

template <int NR, int R>
__device__ __forceinline__ i32x8 ring_pair(FragRing& f) {
  const uint4 x0 = ring_slot<R % NR>(f), x1 = ring_slot<(R + 1) % NR>(f);
  return i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
}

template <int D, int PREC, int M, int MEND = MfmaPlan<D, PREC>::NMFMA>
__device__ __forceinline__ void mfma_steps(MfmaCtx<D, PREC>& c) {
  using P = MfmaPlan<D, PREC>;
  if constexpr (M < MEND) {
    if constexpr (M < P::NS_MFMA) {
      constexpr int st = M / 2, t = M % 2;
      if constexpr (P::F4) {
        const uint4 x = ring_slot<M % P::NR>(c.ring);
        const i32x4 ka = {(int)x.x, (int)x.y, (int)x.z, (int)x.w};
        c.s[t] = rf_mfma_scale_fp4(ka, c.qf4[st], c.s[t], 4, 4, 2 * st, c.ksc[t], 2 * st, c.qsc);
      } else if constexpr (P::QK8) {
        const i32x8 ka = ring_pair<P::NR, 2 * M>(c.ring);
        c.s[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, c.qf8[st], c.s[t], 0, 0, 0,
                                                                 127, 0, 127);
      } else {
        bf16x8 ka;
        __builtin_memcpy(&ka, &ring_slot<M % P::NR>(c.ring), 16);
        c.s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, c.qf[st], c.s[t], 0, 0, 0);
      }
    } else if constexpr (P::VQ && M == P::NS_MFMA + P::NPV) {
      // Row sums: (all-ones 32 x 64) x P^T puts the sum of this lane's query row
      // over the wave's 64 keys in every accumulator value (E4M3 1.0 = 0x38,
      // E2M1 1.0 = 0x2).
      if constexpr (P::F4) {
        constexpr int k1 = 0x22222222;
        const i32x4 ones = {k1, k1, k1, k1};
        c.osum = rf_mfma_scale_fp4(ones, c.pf4, c.osum, 4, 4, 0, 127, 0, c.psc);
      } else {
        constexpr int k1 = 0x38383838;
        const i32x8 ones = {k1, k1, k1, k1, k1, k1, k1, k1};
        c.osum = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, c.pf8, c.osum, 0, 0, 0,
                                                                 127, 0, c.psc);
      }
    } else if constexpr (P::F4) {
      // O^T tile e += V^T (E2M1, scale byte e of vsc) P^T (E2M1, scale psc)
      // over the wave's 64 keys.
      constexpr int e = M - P::NS_MFMA;
      const uint4 x = ring_slot<(P::NS_READ + e) % P::NR>(c.ring);
      const i32x4 va = {(int)x.x, (int)x.y, (int)x.z, (int)x.w};
      c.o[e] = rf_mfma_scale_fp4(va, c.pf4, c.o[e], 4, 4, e, c.vsc, 0, c.psc);
    } else if constexpr (P::VQ) {
      // O^T tile e += 2^(vexp - 127) V^T (E4M3) P^T (E4M3) over the wave's 64 keys.
      constexpr int e = M - P::NS_MFMA;
      const i32x8 va = ring_pair<P::NR, P::NS_READ + 2 * e>(c.ring);
      c.o[e] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, c.pf8, c.o[e], 0, 0, 0, c.vexp,
                                                               0, c.psc);
    } else {
      constexpr int pm = M - P::NS_MFMA, tu = pm / P::DT, e = pm % P::DT;
      constexpr int r = P::NS_READ + pm;
      bf16x8 va;
      __builtin_memcpy(&va, &ring_slot<r % P::NR>(c.ring), 16);
      c.o[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, c.pf16[tu / 2][tu % 2], c.o[e], 0, 0, 0);
    }
    // fp8 S^T products stay first (see pin_products): their results are
    // pinned one product later, so the pin itself waits for nothing.
    if constexpr (P::QK8 && M == P::NS_MFMA) {
      pin_acc(c.s[0]);
      pin_acc(c.s[1]);
    }
    // Refill the slots this product consumed: NR reads stay ahead.
    constexpr int done_before = M == 0 ? 0 : P::rend(M - 1);
    issue_reads<D, PREC, done_before + P::NR, P::rend(M) + P::NR>(c);
    // Keep this order: the scheduler would otherwise pull each read down to
    // its use and leave too few in flight.
    __builtin_amdgcn_sched_barrier(0);
    mfma_steps<D, PREC, M + 1, MEND>(c);
  }
}

// mxfp4 O^T products of the last block (after the loop): one per channel tile,
// the tile index being the opsel immediate of the V^T scale.
template <int D, int PREC, int E = 0>
__device__ __forceinline__ void pv_tail_fp4(MfmaCtx<D, PREC>& c, const uint8_t* vs) {
  if constexpr (E < D / 32) {
    const uint4 x = *reinterpret_cast<const uint4*>(vs + 32 * E * TileGeom<D, PREC>::VSTR);
    const i32x4 va = {(int)x.x, (int)x.y, (int)x.z, (int)x.w};
    c.o[E] = rf_mfma_scale_fp4(va, c.pf4, c.o[E], 4, 4, E, c.vsc, 0, c.psc);
    pv_tail_fp4<D, PREC, E + 1>(c, vs);
  }
}

// Workgroup of 8 waves per (batch, query block, head). Wave w owns query rows
// [32 rg, 32 rg + 32) with rg = w % 4 and key rows [64 kh, 64 kh + 64) of every
// listed block with kh = 1 - w / 4: each wave keeps its own running max / sum /
// O^T over its half of the keys, and the two halves are merged through LDS at
// the end (exact: the merge rescales both to the common maximum).
//
// The two waves that share a SIMD (same rg) run half an iteration apart: the
// kh = 1 group starts one barrier interval late. Each iteration of a wave is
//   MFMA interval: S^T = K Q^T of this block, O^T += V^T P^T of the previous
//                  one, and the global loads of one tile into registers
//   VALU interval: that tile stored to LDS, the softmax of this block's S^T
//                  into P
// so in every interval one wave of each SIMD issues matrix work while the
// other runs the softmax. The MFMA interval streams its LDS operands through
// a ring of fragments kept several reads ahead (the first reads, K of the next
// block, are issued before the barrier that opens it) and spreads its global
// loads between the products. K and V^T tiles are double buffered in LDS: the
// kh = 0 waves copy V^T of the block they are scoring, the kh = 1 waves K of
// the block two ahead. (mxfp4: the kh = 0 waves store that V^T tile in their
// MFMA interval instead, having loaded it one interval earlier.)
//
// Barriers wait only for LDS operations (lds_barrier), and the block ids come
// from a window of list entries held in scalar registers, so no wait in the
// loop covers anything but the data it needs.
//
// ALL (the dense path, no lists) visits every key block in order.
template <int D, int PREC, bool ALL>
__global__ __launch_bounds__(kThreads8, 1) void sparse_attn_kernel(AttnArgs a) {
  using PL = MfmaPlan<D, PREC>;
  using TG = TileGeom<D, PREC>;
  constexpr bool MIX = PL::QK8;           // quantised Q/K (mix, fp8, mxfp4)
  constexpr bool VQ = PL::VQ;             // quantised V and P (fp8, mxfp4)
  constexpr bool F4 = PL::F4;             // E2M1 codes with E8M0 scales (mxfp4)
  constexpr int KROW = TG::KROW;          // K row bytes in global memory
  constexpr int KSTR = TG::KSTR;          // K row stride in LDS (bytes, padded)
  constexpr int VROW = TG::VROW;          // V^T row bytes (128 keys)
  constexpr int VSTR = TG::VSTR;          // V^T row stride in LDS (bytes, padded)
  constexpr int DT = D / 32;              // 32-wide channel tiles of O^T
  constexpr int KCH = KROW / 16;          // 16-byte chunks per K row
  constexpr int VCH = VROW / 16;          // 16-byte chunks per V^T row
  constexpr int K_CH = 128 * KCH / 256;   // K chunks per thread of the kh = 1 group
  constexpr int V_CH = D * VCH / 256;     // V^T chunks per thread of the kh = 0 group
  constexpr int NSTG = K_CH > V_CH ? K_CH : V_CH;
  // mxfp4 (V^T tiles of 8 KiB, two registers of staging per lane): the kh = 0
  // waves store V^T of block i in their MFMA interval, chunk by chunk between
  // the products, each chunk just before its registers take the load of
  // block i + 1 (loaded there one interval earlier, so it has landed), and
  // their softmax interval copies nothing. The other precisions store it in
  // the softmax interval (measured: bf16 +8.5% and mix +4.3% the other way,
  // fp8 unchanged).
  constexpr bool VSL = F4;
  constexpr int KSC = TG::KSC, VSC = TG::VSC;  // mxfp4 scale bytes after each tile
  constexpr int NSC = KSC / 16;           // their 16-byte chunks (K and V alike)
  static_assert(KSC == VSC, "scale chunks");
  constexpr int KT = 128 * KSTR + KSC, VT = D * VSTR + VSC;
  constexpr int TILE_BYTES = 2 * KT + 2 * VT;
  constexpr int MERGE_BYTES = 4 * (DT * 16 + 2) * 64 * 4;
  __shared__ __attribute__((aligned(16)))
  uint8_t smem[TILE_BYTES > MERGE_BYTES ? TILE_BYTES : MERGE_BYTES];
  uint8_t* const kbuf0 = smem;
  uint8_t* const vbuf0 = smem + 2 * KT;

  const RfGeom& g = a.g;
  const int tid = threadIdx.x;
  // The wave index is uniform; readfirstlane lets the compiler see that, so
  // branches on kh are scalar branches.
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, li = lane % 32, h = lane / 32;
  // Waves 4..7 are dispatched later and lose issue and LDS arbitration to
  // waves 0..3 on their SIMD (measured: their MFMA intervals run longer,
  // whatever their role, and s_setprio does not change it). The key half
  // that runs one interval behind goes to the favoured waves 0..3.
  const int rg = wave & 3, kh = (wave >> 2) ^ 1;
  const int gt = tid & 255;  // thread index within its kh group
  int32_t b, q, n;
  decode_wg(g, blockIdx.x, &b, &q, &n);
  const int32_t nk = n / g.G;
  int64_t row0;
  int32_t len;
  rf_block_rows(g, q, &row0, &len);
  const int qrow = 32 * rg + li;
  const bool qvalid = qrow < len;

  MfmaCtx<D, PREC> c;
  // Q fragment (B operand of S^T = K Q^T): query row qrow, channels by k-step.
  float q_sigma = 1.0f;
  if constexpr (F4) {
    // E2M1 codes: channels [64 st + 32 h, +32) are bytes [32 st + 16 h, +16);
    // the row's D/32 scale bytes shifted so that byte 2 st holds block 2 st + h.
    const int64_t qrow_g = ((int64_t)b * g.N1 + n) * g.S + row0 + qrow;
    const uint8_t* qr = a.q8 + qrow_g * (D / 2);
#pragma unroll
    for (int st = 0; st < PL::QK_STEPS; ++st) {
      if (qvalid) {
        const uint4 x = *reinterpret_cast<const uint4*>(qr + 32 * st + 16 * h);
        c.qf4[st] = i32x4{(int)x.x, (int)x.y, (int)x.z, (int)x.w};
      } else {
        c.qf4[st] = i32x4{0, 0, 0, 0};
      }
    }
    const uint8_t* qs = static_cast<const uint8_t*>(a.q_scale) + qrow_g * DT;
    const uint32_t w = !qvalid ? 0u
                       : (DT == 4 ? *reinterpret_cast<const uint32_t*>(qs)
                                  : (uint32_t)*reinterpret_cast<const uint16_t*>(qs));
    c.qsc = (int)(w >> (8 * h));
  } else if constexpr (MIX) {
    const uint8_t* qr = a.q8 + (((int64_t)b * g.N1 + n) * g.S + row0 + qrow) * D;
#pragma unroll
    for (int st = 0; st < PL::QK_STEPS; ++st) {
      if (qvalid) {
        const uint4 x0 = *reinterpret_cast<const uint4*>(qr + 64 * st + 32 * h);
        const uint4 x1 = *reinterpret_cast<const uint4*>(qr + 64 * st + 32 * h + 16);
        c.qf8[st] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                          (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      } else {
        c.qf8[st] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
    q_sigma = static_cast<const float*>(a.q_scale)[((int64_t)b * g.N1 + n) * g.n_blocks + q];
  } else {
    const uint16_t* qr = a.qp + (((int64_t)b * g.N1 + n) * g.S + row0 + qrow) * D;
#pragma unroll
    for (int st = 0; st < PL::QK_STEPS; ++st) {
      if (qvalid) {
        c.qf[st] = *reinterpret_cast<const bf16x8*>(qr + 16 * st + 8 * h);
      } else {
        c.qf[st] = bf16x8{};
      }
    }
  }
  // Let the Q loads land here: otherwise the wait for them stays inside the
  // loop, where it would also wait for the in-flight tile prefetches.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

#pragma unroll
  for (int e = 0; e < DT; ++e) c.o[e] = f32x16{};
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u) c.pf16[t][u] = bf16x8{};
  c.pf8 = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  c.pf4 = i32x4{0, 0, 0, 0};
  c.psc = 127;
  c.vsc = 0;
  c.osum = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  float m_ref = -INFINITY;  // fp8, mxfp4: the reference at which O^T and the row sums are held

  const int64_t sel_row = ((int64_t)b * g.n_blocks + q) * g.N1 + n;
  const list_ptr list = ALL ? nullptr : (list_ptr)(a.select_idx + sel_row * a.max_kv);
  int32_t cnt = ALL ? g.n_blocks : ((list_ptr)a.select_num)[sel_row];
  cnt = cnt < 0 ? 0 : (cnt > a.max_kv ? a.max_kv : cnt);

  const uint8_t* kbytes =
      MIX ? a.k8 + ((int64_t)b * g.N2 + nk) * g.S * KROW
          : reinterpret_cast<const uint8_t*>(a.kp + ((int64_t)b * g.N2 + nk) * g.S * D);
  const uint8_t* vbytes = reinterpret_cast<const uint8_t*>(a.vpt) +
                          ((int64_t)b * g.N2 + nk) * g.n_blocks * (int64_t)D * VROW;
  const scale_ptr kscale =
      MIX && !F4 ? (scale_ptr)(static_cast<const float*>(a.k_scale) + ((int64_t)b * g.N2 + nk) * g.n_blocks)
                 : nullptr;
  const scale_ptr vscale =
      VQ && !F4 ? (scale_ptr)(static_cast<const float*>(a.v_scale) + ((int64_t)b * g.N2 + nk) * g.n_blocks)
                : nullptr;

  // Tile copies: buffer loads over this (batch, kv head)'s K and V^T. Thread
  // gt's chunk m (16 bytes) of a tile of NCH chunks per thread sits at byte
  // 512 NCH (gt / 32) + 16 (gt % 32) + 512 m. The VGPR offset of a load is the
  // tile's first byte plus the thread's part (one add per tile), the
  // instruction immediate is 512 m (< 4096), and the SGPR offset is 0: the
  // hardware checks the VGPR offset plus the immediate against the
  // descriptor's size (the bytes of this (batch, kv head)'s K or V^T) and
  // reads zeros past it, so the tile of a short block at the end of the
  // sequence reads zeros past the sequence and never leaves the buffer.
  const __amdgpu_buffer_rsrc_t rk = raw_buffer(kbytes, (uint32_t)(g.S * KROW));
  const __amdgpu_buffer_rsrc_t rv = raw_buffer(vbytes, (uint32_t)((int64_t)g.n_blocks * D * VROW));
  auto k_tile_off = [&](int32_t jb) -> int {
    int64_t r0;
    int32_t fl;
    rf_block_rows(g, jb, &r0, &fl);
    return (int)(r0 * KROW);
  };
  const int vg_k = (gt >> 5) * (512 * K_CH) + (gt & 31) * 16;
  const int vg_v = (gt >> 5) * (512 * V_CH) + (gt & 31) * 16;
  // mxfp4 scale bytes of this (batch, kv head): K [S][D/32], V [n_blocks][4][D].
  const __amdgpu_buffer_rsrc_t rks =
      F4 ? raw_buffer(static_cast<const uint8_t*>(a.k_scale) + ((int64_t)b * g.N2 + nk) * g.S * DT,
                      (uint32_t)(g.S * DT))
         : raw_buffer(nullptr, 0);
  const __amdgpu_buffer_rsrc_t rvs =
      F4 ? raw_buffer(static_cast<const uint8_t*>(a.v_scale) +
                          ((int64_t)b * g.N2 + nk) * g.n_blocks * (int64_t)VSC,
                      (uint32_t)((int64_t)g.n_blocks * VSC))
         : raw_buffer(nullptr, 0);
  // K rows past a short block's end are the next rows of K, or (past the end
  // of the sequence) zeros; they are masked out of the softmax.
  // (Named registers rather than an array: they must never live in scratch.)
  static_assert(NSTG <= 8, "staging size");
  static_assert(512 * 7 < 4096, "chunk offsets fit the instruction immediate");
  u32x4 st0, st1, st2, st3, st4, st5, st6, st7;
  u32x4 sts;  // mxfp4: one 16-byte chunk of the staged tile's scale bytes
  static_assert(NSC <= 256, "scale chunks per group");
#define RF_GLD1(VAR, M)                                                                    \
  if constexpr ((M) < NSTG) {                                                              \
    if ((M) < nch_) VAR = __builtin_amdgcn_raw_buffer_load_b128(rs_, vo_ + (M) * 512, 0, 0); \
  }
// Chunk slot of thread gt's chunk M in a tile of NCH chunks per thread (the
// byte layout above, in 16-byte units).
#define RF_SLOT(NCH, M) ((gt >> 5) * (32 * (NCH)) + (gt & 31) + 32 * (M))
#define RF_KST1(BUF, VAR, M)                                                               \
  if constexpr ((M) < K_CH) {                                                              \
    const int slot_ = RF_SLOT(K_CH, M), r_ = slot_ / KCH, c_ = slot_ % KCH;                \
    *reinterpret_cast<u32x4*>((BUF) + (VQ ? kslot8(r_) : r_) * KSTR + c_ * 16) = VAR;      \
  }
#define RF_VST1(BUF, VAR, M)                                                               \
  if constexpr ((M) < V_CH) {                                                              \
    const int slot_ = RF_SLOT(V_CH, M), d_ = slot_ / VCH, c_ = slot_ % VCH;                \
    *reinterpret_cast<u32x4*>((BUF) + d_ * VSTR + c_ * 16) = VAR;                          \
  }
// mxfp4 scale chunk: V^T scales copied as they are; K scales of rows
// 16/DT * gt .. (DT bytes each) placed by row like the K rows, in runs of 4
// rows (kslot8 keeps the low two bits of the row).
#define RF_GLDS(RS, SO)                                                                    \
  if constexpr (F4) {                                                                      \
    if (gt < NSC) sts = __builtin_amdgcn_raw_buffer_load_b128((RS), (SO) + gt * 16, 0, 0); \
  }
#define RF_VSST(BUF)                                                                       \
  if constexpr (F4) {                                                                      \
    if (gt < NSC) *reinterpret_cast<u32x4*>((BUF) + D * VSTR + gt * 16) = sts;             \
  }
#define RF_KSST(BUF)                                                                       \
  if constexpr (F4) {                                                                      \
    if (gt < NSC) {                                                                        \
      uint8_t* ks_ = (BUF) + 128 * KSTR;                                                   \
      const int r_ = gt * (16 / DT);                                                       \
      if constexpr (DT == 4) {                                                             \
        *reinterpret_cast<u32x4*>(ks_ + kslot8(r_) * 4) = sts;                             \
      } else {                                                                             \
        *reinterpret_cast<uint2*>(ks_ + kslot8(r_) * 2) = uint2{sts.x, sts.y};             \
        *reinterpret_cast<uint2*>(ks_ + kslot8(r_ + 4) * 2) = uint2{sts.z, sts.w};         \
      }                                                                                    \
    }                                                                                      \
  }
// K tile J (as 16-byte chunks of its row-major bytes) into the staging registers.
#define RF_LOAD_K(J)                                                                       \
  do {                                                                                     \
    const int so_ = k_tile_off(J), nch_ = K_CH, vo_ = vg_k + so_;                          \
    const __amdgpu_buffer_rsrc_t rs_ = rk;                                                 \
    RF_GLD1(st0, 0) RF_GLD1(st1, 1) RF_GLD1(st2, 2) RF_GLD1(st3, 3)                        \
    RF_GLD1(st4, 4) RF_GLD1(st5, 5) RF_GLD1(st6, 6) RF_GLD1(st7, 7)                        \
    RF_GLDS(rks, so_ / KROW * DT)                                                          \
  } while (0)
#define RF_STORE_K(BUF)                                                                    \
  do {                                                                                     \
    RF_KST1(BUF, st0, 0) RF_KST1(BUF, st1, 1) RF_KST1(BUF, st2, 2) RF_KST1(BUF, st3, 3)    \
    RF_KST1(BUF, st4, 4) RF_KST1(BUF, st5, 5) RF_KST1(BUF, st6, 6) RF_KST1(BUF, st7, 7)    \
  } while (0)
#define RF_STORE_V(BUF)                                                                    \
  do {                                                                                     \
    RF_VST1(BUF, st0, 0) RF_VST1(BUF, st1, 1) RF_VST1(BUF, st2, 2) RF_VST1(BUF, st3, 3)    \
    RF_VST1(BUF, st4, 4) RF_VST1(BUF, st5, 5) RF_VST1(BUF, st6, 6) RF_VST1(BUF, st7, 7)    \
  } while (0)

  // Block ids come from a window of four list entries in scalar registers
  // (blocks i .. i + 3); the entry four ahead is loaded one iteration early.
  // An entry outside [0, n_blocks) is processed as a fully masked block
  // (block 0's tiles with no valid key), which adds exactly nothing: the same
  // as skipping it. Entries past the list end stand for block 0 too; nothing
  // reads what is fetched for them.
  const int32_t nbk = g.n_blocks;
  auto entry = [&](int pos) -> int32_t { return pos < cnt ? (ALL ? pos : list[pos]) : -1; };
  auto safe = [&](int32_t jr) -> int32_t { return (jr >= 0 && jr < nbk) ? jr : 0; };
  int32_t w0 = entry(0), w1 = entry(1), w2 = entry(2), w3 = entry(3);

  // Prologue: K of blocks 0 and 1 to LDS. The V^T buffer that
  // the first (empty) PV product reads is zeroed: P is zero there, and
  // 0 * (stale bits) could be NaN.
  if (cnt > 0) {
    if (kh == 0) {
      RF_LOAD_K(safe(w0));
      RF_STORE_K(kbuf0);
      RF_KSST(kbuf0)
    } else {
      RF_LOAD_K(safe(w1));
      RF_STORE_K(kbuf0 + KT);
      RF_KSST(kbuf0 + KT)
    }
    for (int x = tid; x < VT / 16; x += kThreads8)
      reinterpret_cast<uint4*>(vbuf0 + VT)[x] = uint4{0, 0, 0, 0};
    if (VSL && kh == 0) {
      // V^T of block 0, stored in the first MFMA interval.
      const int so_ = safe(w0) * (D * VROW), nch_ = V_CH, vo_ = vg_v + so_;
      const __amdgpu_buffer_rsrc_t rs_ = rv;
      RF_GLD1(st0, 0) RF_GLD1(st1, 1) RF_GLD1(st2, 2) RF_GLD1(st3, 3)
      RF_GLD1(st4, 4) RF_GLD1(st5, 5) RF_GLD1(st6, 6) RF_GLD1(st7, 7)
      RF_GLDS(rvs, safe(w0) * VSC)
    }
  }
  lds_barrier();
  if (kh == 1) lds_barrier();  // the kh = 1 group runs one interval behind

  // This lane's fragment bases: K row 64 kh + kappa(li) (+ 32 t) (fp8: LDS row
  // 64 kh + li (+ 32 t), holding key 64 kh + 16 t + kappa8(li)), V^T row li
  // (+ 32 e) at key column 64 kh + 8 h (+ 16 k-step) (fp8: 64 kh + 32 h).
  // mxfp4: bytes of E2M1, half of fp8's.
  const int krow = VQ ? li : kappa(li);
  const int koff = (64 * kh + krow) * KSTR + (MIX && !F4 ? 32 * h : 16 * h);
  const int voff = F4   ? li * VSTR + 32 * kh + 16 * h
                   : VQ ? li * VSTR + 64 * kh + 32 * h
                        : li * VSTR + 2 * (64 * kh + 8 * h);
  // mxfp4 scale words of a K tile for this lane's rows (LDS rows 64 kh + 32 t
  // + li, as its K fragments), shifted so that byte 2 st is channel block
  // 2 st + h.
  auto read_ksc = [&](const uint8_t* kbuf) {
    if constexpr (F4) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint8_t* p = kbuf + 128 * KSTR + (64 * kh + 32 * t + li) * DT;
        const uint32_t w = DT == 4 ? *reinterpret_cast<const uint32_t*>(p)
                                   : (uint32_t)*reinterpret_cast<const uint16_t*>(p);
        c.ksc[t] = (int)(w >> (8 * h));
      }
    }
  };
  // LDS operations the barrier after the K prefetch leaves in flight: the
  // fragment reads, and (mxfp4) one more for the two scale reads, which the
  // compiler may issue as one instruction or two (either way every earlier
  // store has completed at that count).
  constexpr int NKEEP = PL::NPRE + (F4 ? 1 : 0);
  c.vexp = 127;
  int par = 0;  // parity of block i: its K tile sits in K buffer par
  c.kbase = kbuf0 + koff;
  issue_reads<D, PREC, 0, PL::NPRE>(c);
  read_ksc(kbuf0);
  for (int i = 0; i < cnt; ++i) {
    const int32_t j = safe(w0);
    int64_t kr0;
    int32_t klen;
    rf_block_rows(g, j, &kr0, &klen);
    if (w0 != j) klen = 0;
    // The tile this group loads in this MFMA interval and stores in the VALU
    // interval that follows: V^T of block i, or K of block i + 2.
    const int32_t jcopy = kh == 0 ? (VSL ? safe(w1) : j) : safe(w2);

    // ---- MFMA interval ----
    c.vbase = vbuf0 + (par ^ 1) * VT + voff;  // V^T of the previous block
    if constexpr (F4) {
      // Its scale bytes: quarter 2 kh + h, channels 32 e + li for e < DT.
      const uint8_t* p = vbuf0 + (par ^ 1) * VT + D * VSTR + (2 * kh + h) * D + DT * li;
      c.vsc = DT == 4 ? (int)*reinterpret_cast<const uint32_t*>(p)
                      : (int)*reinterpret_cast<const uint16_t*>(p);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) c.s[t] = f32x16{};
    issue_reads<D, PREC, PL::NPRE, PL::NR>(c);
    // The next tile's global loads ride along with the products, one after
    // every NMFMA / 8 of them, so that no wave stalls on a burst of loads.
    {
      const int so_ = kh == 0 ? jcopy * (D * VROW) : k_tile_off(jcopy);
      const __amdgpu_buffer_rsrc_t rs_ = kh == 0 ? rv : rk;
      const int nch_ = kh == 0 ? V_CH : K_CH;
      const int vo_ = (kh == 0 ? vg_v : vg_k) + so_;
#define RF_Q(K) ((K) * PL::NMFMA / 8)
      uint8_t* const vdst = vbuf0 + par * VT;  // kh = 0: V^T of block i goes here
#define RF_VSL(VAR, M) \
      if (VSL && kh == 0) { RF_VST1(vdst, VAR, M) } \
      RF_GLD1(VAR, M)
      if constexpr (PREC == RF_PREC_MIX) {
        // mix: all loads first (1% faster there; 2.5% slower in bf16 and fp8).
        if (VSL && kh == 0) { RF_VSST(vdst) }
        RF_VSL(st0, 0) RF_VSL(st1, 1) RF_VSL(st2, 2) RF_VSL(st3, 3)
        RF_VSL(st4, 4) RF_VSL(st5, 5) RF_VSL(st6, 6) RF_VSL(st7, 7)
        RF_GLDS(kh == 0 ? rvs : rks, kh == 0 ? jcopy * VSC : so_ / KROW * DT)
        mfma_steps<D, PREC, 0, RF_Q(8)>(c);
      } else {
        mfma_steps<D, PREC, 0, RF_Q(1)>(c);
        RF_VSL(st0, 0)
        mfma_steps<D, PREC, RF_Q(1), RF_Q(2)>(c);
        if (VSL && kh == 0) { RF_VSST(vdst) }
        RF_VSL(st1, 1)
        RF_GLDS(kh == 0 ? rvs : rks, kh == 0 ? jcopy * VSC : so_ / KROW * DT)
        mfma_steps<D, PREC, RF_Q(2), RF_Q(3)>(c);
        RF_VSL(st2, 2)
        mfma_steps<D, PREC, RF_Q(3), RF_Q(4)>(c);
        RF_VSL(st3, 3)
        mfma_steps<D, PREC, RF_Q(4), RF_Q(5)>(c);
        RF_VSL(st4, 4)
        mfma_steps<D, PREC, RF_Q(5), RF_Q(6)>(c);
        RF_VSL(st5, 5)
        mfma_steps<D, PREC, RF_Q(6), RF_Q(7)>(c);
        RF_VSL(st6, 6)
        mfma_steps<D, PREC, RF_Q(7), RF_Q(8)>(c);
        RF_VSL(st7, 7)
      }
#undef RF_VSL
#undef RF_Q
    }
    pin_products(c);
    lds_barrier();

    // ---- VALU interval ----
    // Next window entry (consumed after the closing barrier).
    const int32_t w4 = entry(i + 4 < cnt ? i + 4 : cnt);
    // Tile copy: the staged tile to LDS, then the next one into registers.
    if (kh == 0) {
      if constexpr (!VSL) {
        // V^T of block i into buffer par (read in the next two intervals).
        RF_STORE_V(vbuf0 + par * VT);
        RF_VSST(vbuf0 + par * VT)
      }
    } else {
      // K of block i + 2 into buffer par (block i's K was last read in the
      // MFMA interval just done).
      RF_STORE_K(kbuf0 + par * KT);
      RF_KSST(kbuf0 + par * KT)
    }

    // Mask rows past a short block's end (all rows of a masked block).
    if (klen < 128) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kv = VQ ? 64 * kh + 32 * h + 16 * t + v
                            : 64 * kh + 32 * t + 16 * (v / 8) + 8 * h + (v % 8);
          if (kv >= klen) c.s[t][v] = -INFINITY;
        }
    }

    // mix and fp8 fold the block scales of Q and K into the exponent
    // multiplier; mxfp4 applies its scales inside the products (kscale is not
    // set there).
    float cs = a.scale_log2;
    if constexpr (MIX && !F4) cs *= q_sigma * kscale[j];

    // Maximum of this lane's raw scores; the row maximum over this wave's keys
    // (then the partner half-wave), times cs.
    auto lane_max = [&]() -> float {
      float m0 = c.s[0][0], m1 = c.s[1][0];
#pragma unroll
      for (int v = 1; v < 15; v += 2) {
        m0 = max3f(m0, c.s[0][v], c.s[0][v + 1]);
        m1 = max3f(m1, c.s[1][v], c.s[1][v + 1]);
      }
      return max3f(m0, m1, max3f(c.s[0][15], c.s[1][15], c.s[1][15]));
    };
    auto block_max = [&]() -> float { return max_halves(lane_max()) * cs; };
    // O^T holds every product up to the previous block here, exactly what a
    // rescale of the running state must cover.
    auto rescale = [&](float m_new, float alpha) {
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < DT; ++e)
#pragma unroll
        for (int v = 0; v < 16; ++v) c.o[e][v] *= alpha;
      if constexpr (VQ) {
#pragma unroll
        for (int v = 0; v < 16; ++v) c.osum[v] *= alpha;
      }
    };
    // fp8, mxfp4: move the accumulation reference (O^T and the row sums).
    auto rescale_ref = [&](float new_ref, float alpha) {
      m_ref = new_ref;
#pragma unroll
      for (int e = 0; e < DT; ++e)
#pragma unroll
        for (int v = 0; v < 16; ++v) c.o[e][v] *= alpha;
#pragma unroll
      for (int v = 0; v < 16; ++v) c.osum[v] *= alpha;
    };
    // While every key so far is masked m_run is -inf; any finite stand-in keeps
    // exp2(-inf - m) at 0 instead of NaN.
    auto ref_neg = [&]() -> float { return -fmaxf(m_run, -1e30f); };

    float lsum = 0.0f;
    if constexpr (VQ) {
      // fp8: P = E4M3(2^(t - m_run)) with m_run the exponent of the row's
      // power-of-two block scale, the smallest integer with
      // 2^(max t) <= 448 * 2^m_run over the keys seen so far, raised as soon
      // as a block exceeds it: the largest P stays in (224, 448], and the
      // rescale by a power of two is exact and leaves the rounding of normal P
      // unchanged. mxfp4: P = 2^(t - m_run) in MX blocks of the lane's 32 keys
      // with m_run the integer ceiling of the running maximum (each MX block's
      // own scale absorbs any power of two).
      constexpr float kTop = F4 ? 0.0f : 8.807354922057604f;  // log2(448)
      const float lm = lane_max();
      const float mc = max_halves(lm) * cs - kTop;
      if (__any(mc > m_run)) {
        m_run = fmaxf(m_run, ceilf(mc));
        // O^T and the row sums accumulate at the integer reference m_ref, not
        // at m_run: the products scale P back by 2^(m_run - m_ref) through
        // their P-operand scale, which is exact, so raising m_run costs no
        // rescale. m_ref moves up to m_run (rescaling by that power of two)
        // only at the first finite reference and when the gap exceeds 64
        // binades, far below where the fp32 sums could overflow.
        const bool rebase = m_ref == -INFINITY ? m_run != -INFINITY : m_run - m_ref > 64.0f;
        if (__any(rebase)) {
          const float new_ref = m_run == -INFINITY ? m_ref : m_run;
          rescale_ref(new_ref, m_ref == -INFINITY ? 0.0f : ldexpf(1.0f, (int)(m_ref - new_ref)));
        }
      }
      const int pgap = (m_run == -INFINITY || m_ref == -INFINITY) ? 0 : (int)(m_run - m_ref);
      const float mneg = ref_neg();
      if constexpr (F4) {
        // The lane's MX block: its largest P fixes the exponent e (rf_mx.h);
        // the codes are E2M1 of P / 2^e, taken as 2^(t - m_run - e) (e is an
        // integer, exact in the exponent). Nibble 16 t + v of the B operand
        // is key 32 h + 16 t + v. Row sums: the all-ones product.
        const int ep = rf_mx_scale_exp(__builtin_amdgcn_exp2f(fmaf(lm, cs, mneg)));
        const float mneg_e = mneg - (float)ep;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int t = w / 2, v0 = 8 * (w % 2);
          float p[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) p[x] = __builtin_amdgcn_exp2f(fmaf(c.s[t][v0 + x], cs, mneg_e));
          c.pf4[w] = (int)rf_e2m1_pack8(p);
        }
        c.psc = ep + 127 + pgap;
      } else {
      // P as E4M3 codes (round to nearest even; P <= 448), byte 16 t + v
      // of the B operand. The row sum of the rounded values (what multiplies
      // V) comes from the all-ones product in the next MFMA interval.
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int t = w / 4, v0 = 4 * (w % 4);
        float p[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) p[x] = __builtin_amdgcn_exp2f(fmaf(c.s[t][v0 + x], cs, mneg));
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], pk, true);
        c.pf8[w] = pk;
      }
      c.vexp = (int)((__float_as_uint(vscale[j]) >> 23) & 0xffu);
      c.psc = 127 + pgap;
      }
    } else {
      // bf16 P and fp32 sums hold exponentials far beyond 1, so the reference
      // m_run is only a guard against overflow: the exponentials are taken
      // against the current one, and only if some row's block sum leaves
      // (0, 2^64] (or no key has been seen yet, m_run = -inf) is the block
      // maximum computed, m_run raised to it and the block redone.
      auto exps = [&](float mneg) -> float {
        float ls = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int m = 0; m < 8; ++m) {
              const float p = __builtin_amdgcn_exp2f(fmaf(c.s[t][8 * u + m], cs, mneg));
              ls += p;
              c.pf16[t][u][m] = (__bf16)p;
            }
        return ls;
      };
      lsum = exps(ref_neg());
      if (__any(!(lsum <= 0x1p64f))) {
        const float m_new = fmaxf(m_run, block_max());
        // (m_run = -inf: nothing accumulated yet; alpha 0 also when m_new stays -inf.)
        rescale(m_new, m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new));
        lsum = exps(ref_neg());
      }
    }
    l_run += lsum;

    // First K fragments of block i + 1 (written at least one interval ago,
    // overwritten no earlier than two intervals on): they stay in flight across
    // the barrier, which waits only for this wave's tile stores.
    par ^= 1;
    c.kbase = kbuf0 + par * KT + koff;
    __builtin_amdgcn_sched_barrier(0);
    issue_reads<D, PREC, 0, PL::NPRE>(c);
    read_ksc(kbuf0 + par * KT);
    lds_barrier_keep<NKEEP>();
    w0 = w1;
    w1 = w2;
    w2 = w3;
    w3 = w4;
  }
  // O^T += V^T P^T of the last block.
  if (cnt > 0) {
    const uint8_t* vs = vbuf0 + (par ^ 1) * VT + voff;
    if constexpr (F4) {
      const uint8_t* p = vbuf0 + (par ^ 1) * VT + D * VSTR + (2 * kh + h) * D + DT * li;
      c.vsc = DT == 4 ? (int)*reinterpret_cast<const uint32_t*>(p)
                      : (int)*reinterpret_cast<const uint16_t*>(p);
      pv_tail_fp4<D, PREC>(c, vs);
      constexpr int k1 = 0x22222222;
      const i32x4 ones = {k1, k1, k1, k1};
      c.osum = rf_mfma_scale_fp4(ones, c.pf4, c.osum, 4, 4, 0, 127, 0, c.psc);
    } else if constexpr (VQ) {
#pragma unroll
      for (int e = 0; e < DT; ++e) {
        const uint4 x0 = *reinterpret_cast<const uint4*>(vs + 32 * e * VSTR);
        const uint4 x1 = *reinterpret_cast<const uint4*>(vs + 32 * e * VSTR + 16);
        const i32x8 va = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                          (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        c.o[e] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, c.pf8, c.o[e], 0, 0, 0, c.vexp,
                                                                 0, c.psc);
      }
      constexpr int k1 = 0x38383838;
      const i32x8 ones = {k1, k1, k1, k1, k1, k1, k1, k1};
      c.osum = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, c.pf8, c.osum, 0, 0, 0, 127,
                                                               0, c.psc);
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < DT; ++e) {
            const bf16x8 va = *reinterpret_cast<const bf16x8*>(
                vs + 32 * e * VSTR + 2 * (32 * t + 16 * u));
            c.o[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, c.pf16[t][u], c.o[e], 0, 0, 0);
          }
    }
  }
  if (kh == 0) lds_barrier();  // matches the kh = 1 group's extra barrier
  if constexpr (VQ) {
    l_run = c.osum[0];  // the row sum over this wave's keys (any value)
    m_run = m_ref;      // the reference at which O^T and the row sum are held
  }

#undef RF_LOAD_K
#undef RF_STORE_K
#undef RF_STORE_V
#undef RF_GLD1
#undef RF_SLOT
#undef RF_KST1
#undef RF_VST1
#undef RF_GLDS
#undef RF_VSST
#undef RF_KSST

  __syncthreads();  // every wave is done with the tiles
  // Merge the two key halves: wave (rg, 1) hands its state to wave (rg, 0).
  float* mbuf = reinterpret_cast<float*>(smem) + rg * (DT * 16 + 2) * 64;
  if (kh == 1) {
#pragma unroll
    for (int e = 0; e < DT; ++e)
#pragma unroll
      for (int v = 0; v < 16; ++v) mbuf[(e * 16 + v) * 64 + lane] = c.o[e][v];
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
  // bf16 and mix: each lane summed the keys of its own half-wave, so the row
  // sum adds the partner lane's. fp8: the all-ones product already gave every
  // lane the sum over all the wave's keys.
  if constexpr (!VQ) lt += __shfl_xor(lt, 32);
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
          r[x] = (__bf16)((c.o[e][v] * a0 + mbuf[(e * 16 + v) * 64 + lane] * a1) * inv);
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
                                const uint8_t* k8, const void* q_scale, const void* k_scale,
                                const void* v_scale, const int32_t* select_idx,
                                const int32_t* select_num, int32_t max_kv, void* out_p,
                                void* stream) {
  if (precision != RF_PREC_BF16 && precision != RF_PREC_MIX && precision != RF_PREC_FP8 &&
      precision != RF_PREC_MXFP4)
    return RF_ERR_PRECISION;
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
  a.v_scale = v_scale;
  a.select_idx = select_idx;
  a.select_num = select_num;
  a.max_kv = max_kv;
  a.out_p = static_cast<uint16_t*>(out_p);
  const int64_t wgs = (int64_t)g.B * g.N1 * g.n_blocks;
  if (wgs > 0x7fffffff) return RF_ERR_SHAPE;
  // Tile loads address one (batch, kv head)'s K and V^T through 32-bit buffer
  // offsets.
  const int64_t krow =
      precision == RF_PREC_BF16 ? 2 * g.D : (precision == RF_PREC_MXFP4 ? g.D / 2 : g.D);
  const int64_t vrow =
      precision == RF_PREC_FP8 ? 128 : (precision == RF_PREC_MXFP4 ? 64 : 256);
  if (g.S * krow > 0x7fffffff || (int64_t)g.n_blocks * g.D * vrow > 0x7fffffff) return RF_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((uint32_t)wgs);
  const bool all = select_idx == nullptr;
  // One instantiation per (head_dim, precision, lists or none).
  using Kern = void (*)(AttnArgs);
  static const Kern kernels[2][4][2] = {
      {{sparse_attn_kernel<64, RF_PREC_BF16, false>, sparse_attn_kernel<64, RF_PREC_BF16, true>},
       {sparse_attn_kernel<64, RF_PREC_MIX, false>, sparse_attn_kernel<64, RF_PREC_MIX, true>},
       {sparse_attn_kernel<64, RF_PREC_FP8, false>, sparse_attn_kernel<64, RF_PREC_FP8, true>},
       {sparse_attn_kernel<64, RF_PREC_MXFP4, false>, sparse_attn_kernel<64, RF_PREC_MXFP4, true>}},
      {{sparse_attn_kernel<128, RF_PREC_BF16, false>, sparse_attn_kernel<128, RF_PREC_BF16, true>},
       {sparse_attn_kernel<128, RF_PREC_MIX, false>, sparse_attn_kernel<128, RF_PREC_MIX, true>},
       {sparse_attn_kernel<128, RF_PREC_FP8, false>, sparse_attn_kernel<128, RF_PREC_FP8, true>},
       {sparse_attn_kernel<128, RF_PREC_MXFP4, false>,
        sparse_attn_kernel<128, RF_PREC_MXFP4, true>}}};
  hipLaunchKernelGGL(kernels[g.D == 128][precision][all], grid, dim3(kThreads8), 0, s, a);
  return hipGetLastError() == hipSuccess ? RF_OK : RF_ERR_HIP;
}
