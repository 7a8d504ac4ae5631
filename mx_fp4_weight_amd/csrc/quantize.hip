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

// ---------------------------------------------------------------- NVFP4
// NVFP4 ("Module 11. Speculative Decoding and Quantization" §12): E2M1 values,
// an E4M3 scale per 16 values and one fp32 scale for the tensor. The tensor
// scale is g = amax / (6 · 448) over the finite entries (1 for an all-zero
// tensor); a block's scale is E4M3(amax_block / (6 g)) rounded to nearest, ties
// to the even fraction, saturating at 448; a value is coded from w / (E4M3 · g)
// with the MX-FP4 rounding. Every operation is one correctly rounded fp32
// operation, in that order.

// amax over the finite entries as fp32 bits (non-negative floats order like their bits)
__global__ void nv_clear_kernel(uint32_t* amax_bits) { *amax_bits = 0u; }

__global__ __launch_bounds__(256) void nv_amax_kernel(const float* __restrict__ w, int64_t nvec,
                                                      uint32_t* __restrict__ amax_bits) {
  uint32_t m = 0u;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * blockDim.x) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(w + 4 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t a = v[j] & 0x7fffffffu;
      if (a < 0x7f800000u && a > m) m = a;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t t = __shfl_xor(m, o);
    m = t > m ? t : m;
  }
  // one atomic per workgroup, and only when it can raise the value: thousands of
  // read-modify-writes of one address otherwise serialize in L2
  __shared__ uint32_t wmax[256 / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) wmax[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 1; i < 256 / kWave; ++i) m = wmax[i] > m ? wmax[i] : m;
    if (m != 0u && m > __hip_atomic_load(amax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      atomicMax(amax_bits, m);
  }
}

// in: amax bits; out: g as fp32
__global__ void nv_global_kernel(uint32_t* gbits) {
  const float amax = __uint_as_float(*gbits);
  const float g = amax == 0.0f ? 1.0f : amax / 2688.0f;  // 6 * 448
  *reinterpret_cast<float*>(gbits) = g;
}

// Non-negative fp32 -> E4M3 byte, nearest with ties to the even fraction, saturating at 448.
__device__ inline uint32_t e4m3_rne(float t) {
  if (!(t < 448.0f)) return 0x7Eu;
  const uint32_t b = __float_as_uint(t);
  const int e = (int)(b >> 23) - 127;
  if (e < -6) return (uint32_t)__builtin_rintf(t * 512.0f);  // multiples of 2^-9: 0 .. 8
  const uint32_t mant = b & 0x7fffffu;
  const uint32_t keep = mant >> 20, rem = mant & 0xfffffu;
  const uint32_t up = (rem > 0x80000u) || (rem == 0x80000u && (keep & 1u));
  const uint32_t byte = ((uint32_t)(e + 7) << 3) + keep + up;
  return byte > 0x7Eu ? 0x7Eu : byte;
}

__device__ inline float e4m3_value(uint32_t s) {
  const uint32_t e = (s >> 3) & 15u, m = s & 7u;
  return e == 0u ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// E2M1 code of an already scaled fp32 value: nearest, ties to the even code, saturating at 6.
__device__ inline uint32_t e2m1_code_of(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 31) << 3;
  const float a = fabsf(x);
  uint32_t c = 0;
  c += a > 0.25f;
  c += a >= 0.75f;
  c += a > 1.25f;
  c += a >= 1.75f;
  c += a > 2.5f;
  c += a >= 3.5f;
  c += a > 5.0f;
  return sign | c;
}

// 4 lanes per 16-value block (one 16-byte load each); a lane writes its 4 codes (2 bytes).
__global__ __launch_bounds__(256) void nv_quantize_kernel(const float* __restrict__ w, int64_t nblocks,
                                                          const float* __restrict__ gscale,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales,
                                                          int32_t* __restrict__ flags) {
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = gtid >> 2;
  const int sub = (int)(gtid & 3);
  const bool live = blk < nblocks;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (live) v = *reinterpret_cast<const u32x4*>(w + blk * 16 + sub * 4);
  uint32_t amax = 0;
  int bad = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = v[i] & 0x7fffffffu;
    bad |= a >= 0x7f800000u;
    amax = (a < 0x7f800000u && a > amax) ? a : amax;
  }
#pragma unroll
  for (int o = 1; o < 4; o <<= 1) {
    const uint32_t t = __shfl_xor(amax, o);
    amax = t > amax ? t : amax;
    bad |= __shfl_xor(bad, o);
  }
  const float g = *gscale;
  const float denom = 6.0f * g;
  const uint32_t sbyte = e4m3_rne(__uint_as_float(amax) / denom);
  const float d = e4m3_value(sbyte) * g;
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x = d == 0.0f ? __uint_as_float(v[i] & 0x80000000u) : __uint_as_float(v[i]) / d;
    packed |= e2m1_code_of(x) << (4 * i);
  }
  uint32_t sb = sbyte;
  if (bad) {
    packed = 0;
    sb = 0x7Fu;
  }
  if (live) {
    *reinterpret_cast<uint16_t*>(codes + blk * 8 + sub * 2) = (uint16_t)packed;
    if (sub == 0) scales[blk] = (uint8_t)sb;
  }
  if (__any(live && bad) && (threadIdx.x & (kWave - 1)) == 0) raise_flag(flags, MXS_FLAG_NONFINITE);
}

// ------------------------------------------------- MX activations (W4A8 / W4A4)
// bf16 X[m, k] -> MX-FP8 (E4M3 elements) or MX-FP4 (E2M1) with an E8M0 scale per
// 32 values along k ("Module 11. Speculative Decoding and Quantization" §11 and
// §12: W4A8 / W4A4 quantize the activations too; E4M3 is the 8-bit float with 4
// exponent and 3 fraction bits). Shared exponent as for the weights,
// floor(log2 amax) - emax with emax 8 for E4M3 (448 = 1.75 * 2^8) and 2 for E2M1.

// E4M3 code of v * 2^-e (nearest, ties to the even fraction, saturating at 448, sign
// kept), in integers on the fp32 bit pattern: x = mant * 2^-sh in units of the E4M3
// quantum 2^Q at x's binade (Q = max(E, -6) - 3, E = floor(log2 x)).
__device__ inline uint32_t e4m3_code(uint32_t vbits, int e) {
  const uint32_t sign = (vbits >> 31) << 7;
  const uint32_t a = vbits & 0x7fffffffu;
  if (a == 0u) return sign;
  const int ef = (int)(a >> 23);
  const uint32_t mant = ef ? ((a & 0x7fffffu) | 0x800000u) : (a & 0x7fffffu);
  const int E = floor_log2_bits(a) - e;
  const int Q = (E > -6 ? E : -6) - 3;
  const int sh = 150 + e + Q - (ef ? ef : 1);  // >= 13 for every finite input
  uint32_t q, up;
  if (sh >= 32) {
    q = 0u;
    up = 0u;  // below half a quantum
  } else {
    q = mant >> sh;
    const uint32_t rem = mant & ((1u << sh) - 1u), half = 1u << (sh - 1);
    up = (rem > half) | ((rem == half) & (q & 1u));
  }
  q += up;
  uint32_t byte;
  if (E > -6 || q >= 8u) {
    // normal: q in [8, 16] at exponent E (or the subnormal range rounded up to 2^-6)
    int EE = E > -6 ? E : -6;
    if (q == 16u) {
      q = 8u;
      ++EE;
    }
    byte = ((uint32_t)(EE + 7) << 3) | (q - 8u);
  } else {
    byte = q;  // subnormal: q * 2^-9
  }
  return sign | (byte > 0x7Eu ? 0x7Eu : byte);
}

// 4 lanes per 32-value block, one 16-byte load (8 bf16) each.
// slots (KV cache append): input entry i (per_entry consecutive blocks: one token's heads x
// d/32 blocks) is written at entry slots[i] of the output; a slot outside [0, capacity)
// writes nothing and raises MXS_FLAG_TOKEN_RANGE. Without slots, block b goes to block b.
template <int kFmt>
__global__ __launch_bounds__(256) void quantize_act_kernel(const uint16_t* __restrict__ x, int64_t nblocks,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales,
                                                           int32_t* __restrict__ flags,
                                                           const int32_t* __restrict__ slots = nullptr,
                                                           int64_t per_entry = 1, int64_t capacity = 0) {
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = gtid >> 2;
  const int sub = (int)(gtid & 3);
  bool live = blk < nblocks;
  int64_t oblk = blk;  // output block
  bool out_of_range = false;
  if (slots != nullptr && live) {
    const int64_t entry = blk / per_entry;
    const int64_t slot = slots[entry];
    out_of_range = slot < 0 || slot >= capacity;
    oblk = slot * per_entry + (blk - entry * per_entry);
  }
  u32x4 v = {0u, 0u, 0u, 0u};
  if (live) v = *reinterpret_cast<const u32x4*>(x + blk * 32 + sub * 8);
  uint32_t f[8];  // fp32 bit patterns of the 8 values (element 2i in the low half of word i)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = v[i] << 16;
    f[2 * i + 1] = v[i] & 0xffff0000u;
  }
  uint32_t amax = 0;
  int bad = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t a = f[i] & 0x7fffffffu;
    bad |= a >= 0x7f800000u;
    amax = a > amax ? a : amax;
  }
#pragma unroll
  for (int o = 1; o < 4; o <<= 1) {
    const uint32_t t = __shfl_xor(amax, o);
    amax = t > amax ? t : amax;
    bad |= __shfl_xor(bad, o);
  }
  constexpr int kEmax = kFmt == MXS_ACT_FP8 ? 8 : 2;
  int e = -127;
  if (amax != 0) {
    e = floor_log2_bits(amax) - kEmax;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
  }
  const uint8_t sbyte = bad ? (uint8_t)0xFF : (uint8_t)(e + 127);
  if (kFmt == MXS_ACT_FP8) {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0 |= e4m3_code(f[i], e) << (8 * i);
      w1 |= e4m3_code(f[4 + i], e) << (8 * i);
    }
    if (bad) w0 = w1 = 0u;
    if (live && !out_of_range) *reinterpret_cast<uint2*>(codes + oblk * 32 + sub * 8) = make_uint2(w0, w1);
  } else {
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= e2m1_code(f[i], e) << (4 * i);
    if (bad) packed = 0u;
    if (live && !out_of_range) *reinterpret_cast<uint32_t*>(codes + oblk * 16 + sub * 4) = packed;
  }
  if (live && !out_of_range && sub == 0) scales[oblk] = sbyte;
  if (__any(live && bad && !out_of_range) && (threadIdx.x & (kWave - 1)) == 0) raise_flag(flags, MXS_FLAG_NONFINITE);
  if (__any(live && out_of_range) && (threadIdx.x & (kWave - 1)) == 0) raise_flag(flags, MXS_FLAG_TOKEN_RANGE);
}

}  // namespace

hipError_t launch_quantize_act(const uint16_t* x, int64_t m, int64_t k, int32_t fmt, uint8_t* codes,
                               uint8_t* scales, int32_t* flags, hipStream_t stream) {
  const int64_t nblocks = m * (k / 32);
  const dim3 grid((unsigned)((nblocks * 4 + 255) / 256)), block(256);
  if (fmt == MXS_ACT_FP8)
    quantize_act_kernel<MXS_ACT_FP8><<<grid, block, 0, stream>>>(x, nblocks, codes, scales, flags);
  else
    quantize_act_kernel<MXS_ACT_FP4><<<grid, block, 0, stream>>>(x, nblocks, codes, scales, flags);
  return hipGetLastError();
}

hipError_t launch_kv_append(const uint16_t* kv, int64_t t, int64_t heads, int64_t d, const int32_t* slots,
                            int64_t capacity, uint8_t* codes, uint8_t* scales, int32_t* flags, hipStream_t stream) {
  const int64_t per_entry = heads * (d / 32);
  const int64_t nblocks = t * per_entry;
  const dim3 grid((unsigned)((nblocks * 4 + 255) / 256)), block(256);
  quantize_act_kernel<MXS_ACT_FP4><<<grid, block, 0, stream>>>(kv, nblocks, codes, scales, flags, slots, per_entry,
                                                               capacity);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                           int32_t* flags, hipStream_t stream) {
  const int64_t nblocks = n * (k / 32);
  const int64_t threads = nblocks * 8;
  const int64_t grid = (threads + 255) / 256;
  quantize_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(w, nblocks, codes, scales, flags);
  return hipGetLastError();
}

hipError_t launch_nvfp4_quantize(const float* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                                 float* gscale, int32_t* flags, hipStream_t stream) {
  uint32_t* gbits = reinterpret_cast<uint32_t*>(gscale);
  nv_clear_kernel<<<1, 1, 0, stream>>>(gbits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nvec = n * k / 4;
  int64_t grid = (nvec + 255) / 256;
  grid = grid > 1024 ? 1024 : grid;
  nv_amax_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(w, nvec, gbits);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  nv_global_kernel<<<1, 1, 0, stream>>>(gbits);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t nblocks = n * (k / 16);
  const int64_t threads = nblocks * 4;
  nv_quantize_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream>>>(
      w, nblocks, gscale, codes, scales, flags);
  return hipGetLastError();
}

}  // namespace mxs
