// mxfp4_verify_gemm: Y[m, n] = X[m, k] · Ŵ[n, k]ᵀ over MX-FP4 weights (gfx950).
//
// The verification pass streams every weight once and applies it to all
// m = B·T draft positions ("Module 11. Speculative Decoding and Quantization"
// §4 and §10; the fp32-accumulated MX-FP4 GEMV of the news page "Next-Gen
// Speculative Decoding and FP4 Quantization Shake Up LLM Inference
// Economics", section "Microscaling FP4 (MX-FP4) Integration").
//
// Skinny kernel (m <= 16 per tile). At T = 5 a weight costs 0.53 bytes and 5
// multiply-adds; with one fp32 FMA per product the vector ALUs could not keep
// up with HBM, so the products go to the matrix cores:
//   * the weights are the A operand of v_mfma_f32_16x16x32_bf16 (16 rows × 32 k),
//     decoded in registers by v_cvt_scalef32_pk_bf16_fp4 (two E2M1 nibbles ×
//     2^(s-127) -> two bf16, exact), so the vector ALU does ~0.5 instruction
//     per weight;
//   * the activations are the B operand (32 k × 16 columns, one column per
//     draft position, columns >= m are zero);
//   * a lane loads 16 contiguous code bytes = one whole 32-element MX block of
//     one row, so it needs a single scale byte. The four lanes that share a
//     row read 64 contiguous bytes. The k order inside an MFMA is permuted
//     (lane group g takes block g of a 128-k group, MFMA d takes its 8-element
//     slice d); A and B use the same permutation, so the sum is unchanged.
// A workgroup owns 16 output rows and all of k: its W waves take interleaved
// 128-k groups (neighbouring waves read neighbouring bytes of each row) and
// their partial 16×16 tiles are summed in LDS in wave order, so results are
// deterministic.
#include "common.hpp"
#include "internal.hpp"

namespace mxs {
namespace {

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

constexpr int kMaxWaves = 16;

__global__ __launch_bounds__(kMaxWaves * kWave) void gemm_skinny_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ x, float* __restrict__ y, int n, int k, int m) {
  __shared__ f32x4 red[kMaxWaves][kWave];
  const int W = blockDim.x / kWave;  // waves per workgroup (1..16)
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15;  // A row of this lane; also the B column (draft position)
  const int g = lane >> 4;  // which 32-k block of a 128-k group
  const int row0 = blockIdx.x * 16;
  const int t0 = blockIdx.y * 16;
  const int row = row0 + r;
  const int t = t0 + r;
  const bool row_ok = row < n;
  const bool t_ok = t < m;
  const int kb = k >> 5;               // MX blocks per row
  const int ngroups = (kb + 3) >> 2;   // 128-k groups
  const uint8_t* crow = codes + (size_t)(row_ok ? row : 0) * (size_t)(k >> 1);
  const uint8_t* srow = scales + (size_t)(row_ok ? row : 0) * (size_t)kb;
  const uint16_t* xrow = x + (size_t)(t_ok ? t : 0) * (size_t)k;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int grp = wave; grp < ngroups; grp += W) {
    const int blk = grp * 4 + g;
    const bool blk_ok = blk < kb;
    u32x4 c = {0u, 0u, 0u, 0u};
    uint32_t s = 127u;
    if (row_ok && blk_ok) {
      c = *reinterpret_cast<const u32x4*>(crow + (size_t)blk * 16);
      s = srow[blk];
    }
    u32x4 xb[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) xb[d] = u32x4{0u, 0u, 0u, 0u};
    if (t_ok && blk_ok) {
      const u32x4* xp = reinterpret_cast<const u32x4*>(xrow + (size_t)blk * 32);
#pragma unroll
      for (int d = 0; d < 4; ++d) xb[d] = xp[d];
    }
    const float sf = e8m0_to_f32(s);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const bf16x8 a = decode8(c[d], sf);
      const bf16x8 b = __builtin_bit_cast(bf16x8, xb[d]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
  }

  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 sum = red[0][lane];
    for (int w = 1; w < W; ++w) sum += red[w][lane];
    // lane holds C[4g + i][r]: output row row0 + 4g + i, draft position t0 + r
    if (t_ok) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int orow = row0 + 4 * g + i;
        if (orow < n) y[(size_t)t * (size_t)n + orow] = sum[i];
      }
    }
  }
}

hipError_t launch_w(int waves, const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                    const uint16_t* x, int64_t m, float* y, hipStream_t stream) {
  dim3 grid((unsigned)((n + 15) / 16), (unsigned)((m + 15) / 16));
  gemm_skinny_kernel<<<grid, dim3(waves * kWave), 0, stream>>>(codes, scales, x, y, (int)n, (int)k,
                                                                (int)m);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_gemm(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                              const uint16_t* x, int64_t m, float* y, hipStream_t stream) {
  // waves per workgroup: about 4 groups of 128 k per wave, at most 16 waves
  const int64_t groups = (k / 32 + 3) / 4;
  int waves = (int)(groups / 4);
  waves = waves < 1 ? 1 : (waves > kMaxWaves ? kMaxWaves : waves);
  return launch_w(waves, codes, scales, n, k, x, m, y, stream);
}

}  // namespace mxs
