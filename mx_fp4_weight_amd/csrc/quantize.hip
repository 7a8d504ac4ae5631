// mxfp4_quantize kernel: fp32 W[n, k] -> E2M1 codes [n, k/2] + E8M0 scales [n, k/32].
//
// Format from "Module 11. Speculative Decoding and Quantization" §12 (E2M1
// element, E8M0 power-of-two scale, 32 elements per scale); the shared
// exponent is the OCP MX rule floor(log2 amax) - 2 that the lecture's cited
// MX specification uses, with round-to-nearest-even onto the E2M1 grid and
// saturation at 6.
//
// Mapping: 8 consecutive lanes own one 32-element block (4 floats = one
// 16-byte load per lane), so a wave reads 1 KiB of contiguous input per load
// and writes 2 bytes of codes per lane (128 contiguous bytes per wave). The
// block maximum is combined across the 8 lanes with xor-shuffles.
//
// Rounding is done in integers on the fp32 bit pattern, so it is exact for
// every finite input, subnormals included, whatever the FP denormal mode:
// 4·|v|·2^-e is split into floor q and a "remainder != 0" bit, and compared
// with the doubled-and-doubled midpoints 1, 3, 5, 7, 10, 14, 20 (= 4 × 0.25,
// 0.75, 1.25, 1.75, 2.5, 3.5, 5).
#include "common.hpp"
#include "internal.hpp"

namespace mxs {
namespace {

// floor(log2(a)) for the bit pattern of a positive finite fp32 (subnormals too).
__device__ inline int floor_log2_bits(uint32_t a) {
  const int e = (int)(a >> 23);
  if (e != 0) return e - 127;
  return (31 - __clz(a)) - 149;  // subnormal: value = mantissa * 2^-149
}

// E2M1 code (sign | 3-bit magnitude) of v * 2^-e by round-to-nearest-even with saturation.
__device__ inline uint32_t e2m1_code(uint32_t vbits, int e) {
  const uint32_t sign = (vbits >> 31) << 3;
  const uint32_t a = vbits & 0x7fffffffu;
  const int ef = (int)(a >> 23);
  const uint32_t mant = ef ? ((a & 0x7fffffu) | 0x800000u) : (a & 0x7fffffu);
  // |v| = mant * 2^(max(ef,1) - 150); 4|v| 2^-e = mant * 2^-(sh), sh = 148 + e - max(ef,1) >= 19
  const int sh = 148 + e - (ef ? ef : 1);
  uint32_t q, rem;
  if (sh >= 32) {
    q = 0;
    rem = mant != 0;
  } else {
    q = mant >> sh;
    rem = (mant & ((1u << sh) - 1u)) != 0;
  }
  uint32_t c = 0;
  c += (q > 1u) | ((q == 1u) & rem);    // > 0.25
  c += (q >= 3u);                       // >= 0.75
  c += (q > 5u) | ((q == 5u) & rem);    // > 1.25
  c += (q >= 7u);                       // >= 1.75
  c += (q > 10u) | ((q == 10u) & rem);  // > 2.5
  c += (q >= 14u);                      // >= 3.5
  c += (q > 20u) | ((q == 20u) & rem);  // > 5
  return sign | c;
}

__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ w, int64_t nblocks,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       int32_t* __restrict__ flags) {
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = gtid >> 3;  // 8 lanes per 32-element block
  const int sub = (int)(gtid & 7);
  const bool live = blk < nblocks;

  u32x4 v = {0u, 0u, 0u, 0u};
  if (live) v = *reinterpret_cast<const u32x4*>(w + blk * 32 + sub * 4);

  uint32_t amax = 0;
  int bad = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = v[i] & 0x7fffffffu;
    bad |= a >= 0x7f800000u;  // infinity or NaN
    amax = a > amax ? a : amax;  // positive fp32 bit patterns order like their values
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    const uint32_t t = __shfl_xor(amax, o);
    amax = t > amax ? t : amax;
    bad |= __shfl_xor(bad, o);
  }

  int e = -127;
  if (amax != 0) {
    e = floor_log2_bits(amax) - 2;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
  }
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) packed |= e2m1_code(v[i], e) << (4 * i);
  uint8_t sbyte = (uint8_t)(e + 127);
  if (bad) {
    packed = 0;
    sbyte = 0xFF;
  }
  if (live) {
    *reinterpret_cast<uint16_t*>(codes + blk * 16 + sub * 2) = (uint16_t)packed;
    if (sub == 0) scales[blk] = sbyte;
  }
  // one flag write per wave at most
  if (__any(live && bad) && (threadIdx.x & (kWave - 1)) == 0) raise_flag(flags, MXS_FLAG_NONFINITE);
}

}  // namespace

hipError_t launch_quantize(const float* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                           int32_t* flags, hipStream_t stream) {
  const int64_t nblocks = n * (k / 32);
  const int64_t threads = nblocks * 8;
  const int64_t grid = (threads + 255) / 256;
  quantize_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(w, nblocks, codes, scales, flags);
  return hipGetLastError();
}

}  // namespace mxs
