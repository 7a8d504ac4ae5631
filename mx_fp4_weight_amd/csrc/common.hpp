// Device helpers shared by the gfx950 kernels of the MX-FP4 verification library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxfp4spec.h"

namespace mxs {

constexpr int kWave = 64;  // CDNA wavefront width

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor over [base, base + bytes): loads past the end read zero.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;  // past any num_records: the load reads 0

// A buffer-load offset passed through an empty asm. Without it the compiler folds an
// unrolled step's constant into the load's immediate field and branches around the
// load on its validity select, and a load on one side of a branch makes the later
// wait counts conservative (waiting for loads just issued).
__device__ inline uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Workgroup barrier that orders LDS accesses only (global loads stay in flight).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt immediate that waits until at most n (< 64) vector memory operations
// are outstanding and leaves the export and LDS/scalar counters alone: vmcnt bits
// [3:0] and [15:14], expcnt [6:4] = 7, lgkmcnt [11:8] = 15.
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// OR a device-detected condition into the caller's flag word (vector atomic).
__device__ inline void raise_flag(int32_t* flags, int32_t bit) {
  if (flags) atomicOr(flags, bit);
}

// exp(d) in fp64 for d <= 0 (d = -inf gives 0), relative error below 1e-14.
// Cody–Waite reduction d = k ln2 + r with |r| <= ln2/2, then a degree-12
// Taylor polynomial of e^r in Horner form and a scale by 2^k. The same steps
// hold for positive d up to 709 (k <= 1023; the two-part ln 2 keeps k ln2
// exact for |k| < 2^20), which the selection's masses against 0 use.
__device__ inline double exp_neg_f64(double d) {
  if (!(d > -745.0)) return 0.0;  // also catches -inf; NaN never reaches here
  const double kLog2e = 1.4426950408889634;
  const double kLn2Hi = 6.93147180369123816490e-01;
  const double kLn2Lo = 1.90821492927058770002e-10;
  double k = __builtin_rint(d * kLog2e);
  double r = __builtin_fma(-k, kLn2Hi, d);
  r = __builtin_fma(-k, kLn2Lo, r);
  // 1/n! for n = 12 .. 1
  double p = 2.08767569878680989792e-09;
  p = __builtin_fma(p, r, 2.50521083854417187751e-08);
  p = __builtin_fma(p, r, 2.75573192239858906526e-07);
  p = __builtin_fma(p, r, 2.75573192239858906526e-06);
  p = __builtin_fma(p, r, 2.48015873015873015873e-05);
  p = __builtin_fma(p, r, 1.98412698412698412698e-04);
  p = __builtin_fma(p, r, 1.38888888888888888889e-03);
  p = __builtin_fma(p, r, 8.33333333333333333333e-03);
  p = __builtin_fma(p, r, 4.16666666666666666667e-02);
  p = __builtin_fma(p, r, 1.66666666666666666667e-01);
  p = __builtin_fma(p, r, 0.5);
  p = __builtin_fma(p, r, 1.0);
  p = __builtin_fma(p, r, 1.0);
  return __builtin_ldexp(p, (int)k);
}

// 2^(j/32), j = 0..31, each correctly rounded to fp64 (computed to 60 digits).
constexpr double kExp2Table32[32] = {
    0x1.0000000000000p+0, 0x1.059b0d3158574p+0, 0x1.0b5586cf9890fp+0, 0x1.11301d0125b51p+0,
    0x1.172b83c7d517bp+0, 0x1.1d4873168b9aap+0, 0x1.2387a6e756238p+0, 0x1.29e9df51fdee1p+0,
    0x1.306fe0a31b715p+0, 0x1.371a7373aa9cbp+0, 0x1.3dea64c123422p+0, 0x1.44e086061892dp+0,
    0x1.4bfdad5362a27p+0, 0x1.5342b569d4f82p+0, 0x1.5ab07dd485429p+0, 0x1.6247eb03a5585p+0,
    0x1.6a09e667f3bcdp+0, 0x1.71f75e8ec5f74p+0, 0x1.7a11473eb0187p+0, 0x1.82589994cce13p+0,
    0x1.8ace5422aa0dbp+0, 0x1.93737b0cdc5e5p+0, 0x1.9c49182a3f090p+0, 0x1.a5503b23e255dp+0,
    0x1.ae89f995ad3adp+0, 0x1.b7f76f2fb5e47p+0, 0x1.c199bdd85529cp+0, 0x1.cb720dcef9069p+0,
    0x1.d5818dcfba487p+0, 0x1.dfc97337b9b5fp+0, 0x1.ea4afa2a490dap+0, 0x1.f50765b6e4540p+0,
};

// exp(d) in fp64 for d <= 0 (d = -inf gives 0), relative error below 1e-14, by the
// table-driven method of P. T. P. Tang (ACM TOMS 15(2), 1989): d = (32m + j) ln2/32 + r
// with |r| <= ln2/64 (the same two-part ln 2 split as above, scaled by 1/32), then
// e^d = 2^m * 2^(j/32) * p(r) with p the degree-5 Taylor polynomial of e^r (truncation
// below 2.3e-15 relative). tab holds kExp2Table32 (in LDS: the index differs per lane).
// About two thirds of the fp64 operations of exp_neg_f64.
__host__ __device__ inline double exp_neg_f64_tab(double d, const double* tab) {
  if (!(d > -745.0)) return 0.0;
  const double kInvL = 46.166241308446828;  // 32 / ln 2
  const double kL1 = 6.93147180369123816490e-01 / 32.0;
  const double kL2 = 1.90821492927058770002e-10 / 32.0;
  const double nd = __builtin_rint(d * kInvL);
  double r = __builtin_fma(-nd, kL1, d);
  r = __builtin_fma(-nd, kL2, r);
  const int n = (int)nd;
  double p = 8.33333333333333333333e-03;  // 1/5!
  p = __builtin_fma(p, r, 4.16666666666666666667e-02);
  p = __builtin_fma(p, r, 1.66666666666666666667e-01);
  p = __builtin_fma(p, r, 0.5);
  p = __builtin_fma(p, r, 1.0);
  p = __builtin_fma(p, r, 1.0);
  return __builtin_ldexp(tab[n & 31] * p, n >> 5);
}

// NaN or +inf, in one class test (v_cmp_class_f32, class bits: signalling NaN, quiet NaN, +inf).
__device__ inline bool nan_or_pinf(float x) { return __builtin_amdgcn_classf(x, 0x203); }

// The non-inline constants of exp_neg_f64_tab, held in registers. exp_consts() passes them
// through an empty asm statement, so the compiler cannot rebuild them before every use (it
// otherwise copies a constant into the accumulator of each Horner step: about six vector moves
// per exponential). Same operations, same order: bit-identical results.
struct ExpK {
  double inv_l, l1, l2, c5, c4, c3;
};
__device__ inline ExpK exp_consts() {
  ExpK k{46.166241308446828, 6.93147180369123816490e-01 / 32.0, 1.90821492927058770002e-10 / 32.0,
         8.33333333333333333333e-03, 4.16666666666666666667e-02, 1.66666666666666666667e-01};
  asm volatile("" : "+v"(k.inv_l), "+v"(k.l1), "+v"(k.l2), "+v"(k.c5), "+v"(k.c4), "+v"(k.c3));
  return k;
}
__device__ inline double exp_neg_f64_tab(double d, const double* tab, const ExpK& k) {
  if (!(d > -745.0)) return 0.0;
  const double nd = __builtin_rint(d * k.inv_l);
  double r = __builtin_fma(-nd, k.l1, d);
  r = __builtin_fma(-nd, k.l2, r);
  const int n = (int)nd;
  double p = k.c5;
  p = __builtin_fma(p, r, k.c4);
  p = __builtin_fma(p, r, k.c3);
  p = __builtin_fma(p, r, 0.5);
  p = __builtin_fma(p, r, 1.0);
  p = __builtin_fma(p, r, 1.0);
  return __builtin_ldexp(tab[n & 31] * p, n >> 5);
}

// Lane exchanges inside a wave. DPP moves (a VALU operand modifier, no LDS trip) cover the
// steps inside each 16-lane row: swaps within groups of four, then rotations of the row by 4
// and 8; the two steps across rows (16, 32) go through ds_bpermute.
constexpr int kDppQuadXor1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);  // lane ^ 1
constexpr int kDppQuadXor2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);  // lane ^ 2
constexpr int kDppRowRor4 = 0x124;                                 // rotate the row by 4
constexpr int kDppRowRor8 = 0x128;                                 // rotate the row by 8
template <int kCtrl>
__device__ inline int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}
template <int kCtrl>
__device__ inline float dpp_f32(float v) {
  return __int_as_float(dpp_i32<kCtrl>(__float_as_int(v)));
}
template <int kCtrl>
__device__ inline double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)dpp_i32<kCtrl>((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)dpp_i32<kCtrl>((int)(uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Wave-wide reductions (every lane of the wave active). wave_max and wave_or give every lane
// the result; wave_sum_f64 adds in a fixed order and the result of lane 0 is the one to use
// (other lanes may differ in the last bit).
__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRowRor4>(v));
  v = fmaxf(v, dpp_f32<kDppRowRor8>(v));
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ inline int wave_or(int v) {
  v |= dpp_i32<kDppQuadXor1>(v);
  v |= dpp_i32<kDppQuadXor2>(v);
  v |= dpp_i32<kDppRowRor4>(v);
  v |= dpp_i32<kDppRowRor8>(v);
  v |= __shfl_xor(v, 16);
  return v | __shfl_xor(v, 32);
}
__device__ inline double wave_sum_f64(double v) {
  v += dpp_f64<kDppQuadXor1>(v);
  v += dpp_f64<kDppQuadXor2>(v);
  v += dpp_f64<kDppRowRor4>(v);
  v += dpp_f64<kDppRowRor8>(v);
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// Inclusive fp64 scan over the wave in lane order (every lane active): shifts of 1, 2, 4, 8
// inside each 16-lane row (DPP, lanes before the row start add 0), then each row adds the
// totals of the rows before it, read from lanes 15, 31 and 47 and added in row order. The
// order of the additions is fixed, so the same inputs give the same outputs.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
__device__ inline double readlane_f64(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ inline double wave_inclusive_scan_f64(double v) {
  v += dpp_f64<kDppRowShr1>(v);
  v += dpp_f64<kDppRowShr2>(v);
  v += dpp_f64<kDppRowShr4>(v);
  v += dpp_f64<kDppRowShr8>(v);
  const double r0 = readlane_f64(v, 15), r1 = readlane_f64(v, 31), r2 = readlane_f64(v, 47);
  const int row = (int)(threadIdx.x & (kWave - 1)) >> 4;
  double base = row >= 1 ? r0 : 0.0;
  base = row >= 2 ? base + r1 : base;
  base = row >= 3 ? base + r2 : base;
  return base + v;
}

// Block-wide reductions through LDS for blockDim.x == kThreads (a multiple of 64).
template <int kThreads>
__device__ inline float block_max(float v, float* lds) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) lds[w] = v;
  __syncthreads();
  float r = lds[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) r = fmaxf(r, lds[i]);
  __syncthreads();
  return r;
}

// block_max of m and block_or of f in one round of barriers.
template <int kThreads>
__device__ inline void block_max_or(float& m, int& f, float* lds_f, int* lds_i) {
  m = wave_max(m);
  f = wave_or(f);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    lds_f[w] = m;
    lds_i[w] = f;
  }
  __syncthreads();
  float r = lds_f[0];
  int o = lds_i[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) {
    r = fmaxf(r, lds_f[i]);
    o |= lds_i[i];
  }
  __syncthreads();
  m = r;
  f = o;
}

// Deterministic fp64 block sum: a fixed order inside each wave (lane 0's total), then the
// wave totals in wave order.
template <int kThreads>
__device__ inline double block_sum_f64(double v, double* lds) {
  v = wave_sum_f64(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) lds[w] = v;
  __syncthreads();
  double r = lds[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) r += lds[i];
  __syncthreads();
  return r;
}

template <int kThreads>
__device__ inline int block_or(int v, int* lds) {
  v = wave_or(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) lds[w] = v;
  __syncthreads();
  int r = lds[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) r |= lds[i];
  __syncthreads();
  return r;
}

// Inclusive fp64 scan of one value per thread over the block, in thread order:
// wave_inclusive_scan_f64 inside each wave, then the exclusive prefix of the wave
// totals. Same inputs always give bit-identical outputs.
template <int kThreads>
__device__ inline double block_inclusive_scan_f64(double v, double* lds) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  v = wave_inclusive_scan_f64(v);
  if (lane == kWave - 1) lds[w] = v;
  __syncthreads();
  double base = 0.0;
#pragma unroll
  for (int i = 0; i < kThreads / kWave; ++i)
    if (i < w) base += lds[i];
  __syncthreads();
  return base + v;
}

// Two block_inclusive_scan_f64 at once (the same arithmetic for each value, so each result is
// bit-identical to its own call; the two chains overlap). lds: 2 * kThreads / kWave.
template <int kThreads>
__device__ inline void block_inclusive_scan2_f64(double& a, double& b, double* lds) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  a = wave_inclusive_scan_f64(a);
  b = wave_inclusive_scan_f64(b);
  if (lane == kWave - 1) {
    lds[w] = a;
    lds[kThreads / kWave + w] = b;
  }
  __syncthreads();
  double base_a = 0.0, base_b = 0.0;
#pragma unroll
  for (int i = 0; i < kThreads / kWave; ++i)
    if (i < w) {
      base_a += lds[i];
      base_b += lds[kThreads / kWave + i];
    }
  __syncthreads();
  a = base_a + a;
  b = base_b + b;
}

}  // namespace mxs
