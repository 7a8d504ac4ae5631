// mxfp4_verify_gemm: Y[m, n] = X[m, k] · Ŵ[n, k]ᵀ over MX-FP4 weights (gfx950).
//
// The verification pass streams every weight once and applies it to all
// m = B·T draft positions ("Module 11. Speculative Decoding and Quantization"
// §4 and §10; the fp32-accumulated MX-FP4 GEMV of the news page "Next-Gen
// Speculative Decoding and FP4 Quantization Shake Up LLM Inference
// Economics", section "Microscaling FP4 (MX-FP4) Integration").
//
// Skinny kernel (m <= 16 per column tile). At T = 5 a weight costs 0.53 bytes
// and 5 multiply-adds; one fp32 FMA per product would need ~5 vector
// instructions per weight, more than the vector ALUs can issue at HBM speed,
// so the products go to the matrix cores:
//   * the weights are the A operand of v_mfma_f32_16x16x32_bf16 (16 rows × 32 k),
//     decoded in registers by v_cvt_scalef32_pk_bf16_fp4 (two E2M1 nibbles ×
//     2^(s-127) -> two bf16, exact): ~0.56 vector instructions per weight;
//   * the activations are the B operand (32 k × 16 columns, one column per
//     draft position; columns >= m are zero and their lanes load nothing);
//   * a lane loads 16 contiguous code bytes = one whole 32-element MX block of
//     one row, so it needs one scale byte. The four lanes of a row read 64
//     contiguous bytes. Inside an MFMA the k order is permuted (lane group g
//     takes block g of a 128-k group, MFMA d takes slice d of every block); A
//     and B use the same permutation, so the sum is unchanged.
//
// Work split: a workgroup owns R×16 output rows and all of k; its W waves own
// contiguous k-slices of `gpw` 128-k groups. A wave walks its slice S groups
// at a time and issues the loads of the next S groups before the MFMAs of the
// current ones (register double buffering), so each wave keeps R·S 1 KiB code
// loads in flight. The activations of a group are loaded once per wave and
// reused by its R row tiles. Partial 16×16 tiles are summed across waves in
// LDS in wave order: results are deterministic.
#include "common.hpp"
#include "internal.hpp"

namespace mxs {
namespace {

constexpr int kMaxWaves = 8;  // 8 waves = 2 per SIMD, so a wave may use up to 256 registers

// E8M0 byte -> fp32 scale operand 2^(s-127): s << 23 is exactly the fp32 with
// that exponent; byte 0 (2^-127) is the subnormal 0x00400000; byte 255 is NaN.
__device__ inline float e8m0_to_f32(uint32_t s) {
  uint32_t bits = s << 23;
  bits = (s == 0u) ? 0x00400000u : bits;
  bits = (s == 255u) ? 0x7fc00000u : bits;
  return __uint_as_float(bits);
}

// Eight E2M1 codes (one 32-bit word, element j in nibble j) × scale -> 8 bf16.
__device__ inline bf16x8 decode8(uint32_t c, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 3);
  bf16x8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

template <int R, int S>
struct Stage {
  u32x4 c[R][S];     // 16 code bytes (one MX block) per row tile and group
  uint32_t s[R][S];  // its scale byte
  u32x4 xb[S][4];    // activations: 4 × 8 bf16 per group
};

template <int R, int S>
__global__ __launch_bounds__(kMaxWaves * kWave) void gemm_skinny_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ x, float* __restrict__ y, int n, int k, int m, int gpw,
    int y_vec4) {
  extern __shared__ f32x4 red[];  // [W][R][64]
  const int W = blockDim.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15;  // A row of this lane inside a tile; also its B column
  const int g = lane >> 4;  // which 32-k block of a 128-k group
  const int row_base = blockIdx.x * (16 * R);
  const int t = blockIdx.y * 16 + r;
  const bool t_ok = t < m;
  const int kb = k >> 5;
  const int ngroups = (kb + 3) >> 2;
  const int gs = wave * gpw;
  const int ge = min(ngroups, gs + gpw);

  const uint8_t* crow[R];
  const uint8_t* srow[R];
  bool rok[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int row = row_base + 16 * i + r;
    rok[i] = row < n;
    const size_t rr = (size_t)(rok[i] ? row : 0);
    crow[i] = codes + rr * (size_t)(k >> 1);
    srow[i] = scales + rr * (size_t)kb;
  }
  const uint16_t* xrow = x + (size_t)(t_ok ? t : 0) * (size_t)k;

  auto load = [&](int gbase, Stage<R, S>& st) {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const int blk = (gbase + j) * 4 + g;
      const bool ok = (gbase + j) < ge && blk < kb;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        st.c[i][j] = u32x4{0u, 0u, 0u, 0u};
        st.s[i][j] = 127u;
        if (ok && rok[i]) {
          st.c[i][j] = *reinterpret_cast<const u32x4*>(crow[i] + (size_t)blk * 16);
          st.s[i][j] = srow[i][blk];
        }
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) st.xb[j][d] = u32x4{0u, 0u, 0u, 0u};
      if (ok && t_ok) {
        const u32x4* xp = reinterpret_cast<const u32x4*>(xrow + (size_t)blk * 32);
#pragma unroll
        for (int d = 0; d < 4; ++d) st.xb[j][d] = xp[d];
      }
    }
  };

  f32x4 acc[R];
#pragma unroll
  for (int i = 0; i < R; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Stage<R, S>& st) {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      float sf[R];
#pragma unroll
      for (int i = 0; i < R; ++i) sf[i] = e8m0_to_f32(st.s[i][j]);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, st.xb[j][d]);
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const bf16x8 a = decode8(st.c[i][j][d], sf[i]);
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
        }
      }
    }
  };

  if (gs < ge) {
    Stage<R, S> cur;
    load(gs, cur);
    for (int gb = gs; gb < ge; gb += S) {
      Stage<R, S> nxt;
      const bool more = gb + S < ge;
      if (more) load(gb + S, nxt);
      compute(cur);
      if (more) cur = nxt;
    }
  }

#pragma unroll
  for (int i = 0; i < R; ++i) red[(wave * R + i) * kWave + lane] = acc[i];
  __syncthreads();
  // wave w sums tile w, w + W, ... over all waves in wave order
  for (int i = wave; i < R; i += W) {
    f32x4 sum = red[i * kWave + lane];
    for (int w = 1; w < W; ++w) sum += red[(w * R + i) * kWave + lane];
    // lane holds C[4g + e][r]: output row row_base + 16 i + 4 g + e, position t
    const int orow = row_base + 16 * i + 4 * g;
    if (t_ok) {
      float* yp = y + (size_t)t * (size_t)n + orow;
      if (y_vec4 && orow + 3 < n) {
        *reinterpret_cast<f32x4*>(yp) = sum;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (orow + e < n) yp[e] = sum[e];
      }
    }
  }
}

template <int R, int S>
hipError_t launch_rs(int waves, int gpw, const uint8_t* codes, const uint8_t* scales, int64_t n,
                     int64_t k, const uint16_t* x, int64_t m, float* y, hipStream_t stream) {
  dim3 grid((unsigned)((n + 16 * R - 1) / (16 * R)), (unsigned)((m + 15) / 16));
  const size_t lds = sizeof(f32x4) * (size_t)waves * R * kWave;
  // 16-byte stores of 4 consecutive outputs need n % 4 == 0 and a 16-byte aligned y
  const int y_vec4 = (n % 4 == 0) && ((reinterpret_cast<uintptr_t>(y) & 15) == 0);
  gemm_skinny_kernel<R, S><<<grid, dim3(waves * kWave), lds, stream>>>(
      codes, scales, x, y, (int)n, (int)k, (int)m, gpw, y_vec4);
  return hipGetLastError();
}

struct Config {
  int R, S, gpw;
};

hipError_t launch_cfg(Config c, const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                      const uint16_t* x, int64_t m, float* y, hipStream_t stream) {
  const int ngroups = (int)((k / 32 + 3) / 4);
  int gpw = c.gpw < 1 ? 1 : c.gpw;
  int waves = (ngroups + gpw - 1) / gpw;
  if (waves > kMaxWaves) {  // widen the slices until the workgroup fits
    gpw = (ngroups + kMaxWaves - 1) / kMaxWaves;
    waves = (ngroups + gpw - 1) / gpw;
  }
#define MXS_RS(RR, SS) \
  if (c.R == RR && c.S == SS) return launch_rs<RR, SS>(waves, gpw, codes, scales, n, k, x, m, y, stream);
  MXS_RS(1, 1) MXS_RS(1, 2) MXS_RS(1, 4) MXS_RS(2, 1) MXS_RS(2, 2) MXS_RS(2, 4)
  MXS_RS(4, 1) MXS_RS(4, 2)
#undef MXS_RS
  return hipErrorInvalidValue;
}

// Shape-based choice: enough waves in flight to cover HBM latency on 256 CUs.
Config choose(int64_t n, int64_t k) {
  const int64_t ngroups = (k / 32 + 3) / 4;
  Config c{1, 2, 4};
  if (n >= 8192) c.R = 2;
  if (ngroups <= 8) c.gpw = 2;
  return c;
}

}  // namespace

hipError_t launch_verify_gemm(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                              const uint16_t* x, int64_t m, float* y, hipStream_t stream) {
  return launch_cfg(choose(n, k), codes, scales, n, k, x, m, y, stream);
}

#ifdef MXS_TUNING
hipError_t launch_verify_gemm_cfg(int R, int S, int gpw, const uint8_t* codes,
                                  const uint8_t* scales, int64_t n, int64_t k, const uint16_t* x,
                                  int64_t m, float* y, hipStream_t stream) {
  return launch_cfg(Config{R, S, gpw}, codes, scales, n, k, x, m, y, stream);
}
#endif

}  // namespace mxs

#ifdef MXS_TUNING
// Tuning builds only (not part of the product library): explicit tile configuration.
extern "C" int mxs_tune_verify_gemm(const uint8_t* codes, const uint8_t* scales, int64_t n,
                                    int64_t k, const uint16_t* x, int64_t m, float* y, int R, int S,
                                    int gpw, void* stream) {
  return (int)mxs::launch_verify_gemm_cfg(R, S, gpw, codes, scales, n, k, x, m, y,
                                          static_cast<hipStream_t>(stream));
}
#endif
