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
#include <atomic>
#include <type_traits>

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

// E4M3 scale byte (NVFP4 block scale) -> fp32: bias 7, exponent 0 subnormal (m·2^-9),
// S.1111.111 NaN. Exact.
__device__ inline float e4m3_to_f32(uint32_t s) {
  const uint32_t e = (s >> 3) & 15u, m = s & 7u;
  float v = e == 0u ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  v = (e == 15u && m == 7u) ? __uint_as_float(0x7fc00000u) : v;
  return (s & 0x80u) ? -v : v;
}

// Eight E2M1 codes × an arbitrary fp32 block scale -> 8 bf16. The conversion
// instruction applies only the power-of-two part of its scale operand, so the
// codes are decoded at scale 1 into fp32, multiplied by the scale (E2M1 × E4M3
// has at most 6 significant bits: exact) and packed to bf16 (exact as well).
__device__ inline bf16x8 decode8_scaled(uint32_t c, float scale) {
  bf16x8 r;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    f32x2 f;
    if (h == 0) f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
    else if (h == 1) f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
    else if (h == 2) f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
    else f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
    r[2 * h] = (__bf16)(f[0] * scale);
    r[2 * h + 1] = (__bf16)(f[1] * scale);
  }
  return r;
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

// ---------------------------------------------------------------------------
// Main kernel: persistent workgroups, activations staged once in LDS.
//
// A workgroup stages X[t0 : t0+mt, :] into LDS once, then walks row blocks
// rb = blockIdx.x, blockIdx.x + gridDim.x, ... Inside a row block (R×16 rows,
// all of k) wave w owns the contiguous k-slice of G groups starting at w·G and
// issues all of its R·G code loads (1 KiB each per wave) plus the scale loads
// at once. While a row block is computed, the loads of the next one are
// already in flight (two register buffers, loop unrolled by two so no copy
// forces a wait). Loads go through buffer descriptors that cover exactly the
// valid bytes of a row block: rows past n, groups past the slice and a
// missing next block read as zero without a branch, so the compiler's
// wait counts stay exact. Partial tiles are reduced in LDS (two buffers
// alternate between row blocks) behind an LDS-only barrier, which leaves the
// prefetched global loads in flight.

// X staged in LDS in MFMA-operand order. The 16-byte chunk q (8 bf16) of
// activation row t goes to unit ((grp*4 + d)*mt + t)*4 + g with grp = q/16,
// g = (q/4)%4, d = q%4: for one group and MFMA slice d, the lanes (t, g) read
// consecutive 16-byte units, so ds_read_b128 has no bank conflicts.
__device__ inline int xunit(int grp, int d, int t, int g, int mt) { return ((grp * 4 + d) * mt + t) * 4 + g; }

// kNv: NVFP4 weights (an E4M3 scale per 16 values: 32 scale bytes per 4 groups of a row)
// instead of MX-FP4 (an E8M0 scale per 32 values: 16 bytes per 4 groups).
// kTiled (G = 4): codes in the 1 KiB (16 rows x 128 k) tile layout and, for MX-FP4, scales
// in the 2 KiB (128 rows x 512 k) window layout (NVFP4 scales stay in the row layout). A unit's code load of one row tile and group
// then reads 1 KiB contiguously (64 bytes of each of 16 rows otherwise), and its scale
// load 256 bytes. Every unit's 4 groups are one 512-k window: slices and phases start on
// multiples of 4 groups.
template <int R, int G, bool kNv>
struct Block {
  u32x4 c[R][G];                      // 16 code bytes per row tile and group
  u32x4 s[R][kNv ? G / 2 : G / 4];    // scale bytes of the row for these groups
};

// Up to kMaxGroup independent products with the same k and m share one launch
// (the projections of one layer that read the same input, or any independent
// set): the persistent grid is split between them in proportion to their row
// blocks, so a workgroup stages one problem's activations once.
constexpr int kMaxGroup = 8;

struct Problem {
  const uint8_t* codes;
  const uint8_t* scales;
  const uint16_t* x;
  float* y;
  const float* gscale;  // NVFP4 tensor scale (device), null for MX-FP4
  int n, nrb, y_vec4;
  int brows;            // rows per row block: 16·R, or 8 (R = 1: the MFMA's upper 8 rows read zeros)
};

struct Group {
  Problem p[kMaxGroup];
  int wg_start[kMaxGroup + 1];  // workgroups [wg_start[i], wg_start[i+1]) serve problem i
  int count;
};

// nred: partial-tile buffers for the cross-wave sum: 2 alternate between row blocks,
// 1 when that is what lets the targeted number of workgroups share a CU's LDS.
// kPair (several phases only): a workgroup owns the row blocks wg and wg + ngrid (ngrid:
// the product's workgroups) and walks them phase by phase (phase 0 of both, then phase 1 of both, ...), with a
// second set of accumulators, so a phase's activations are staged once for two row
// blocks and every workgroup is resident at once.
// kStream: the weight codes and scales are loaded non-temporally (the cache policy of a stream
// read once: measured 3-8% faster per launch than the default policy). Used when every weight is
// read by one workgroup only (m <= 16: one position tile); with several position tiles the
// workgroups of a row block read the same weights and the default policy keeps them in L2.
template <int R, int G, int D, bool kNv, bool kPair = false, bool kTiled = false, bool kStream = false>
__global__ __launch_bounds__(kMaxWaves * kWave) void gemm_skinny_kernel(const Group grp, int k, int m,
                                                                         int nsub, int phases,
                                                                         int ngroups_p, int nred) {
  static_assert(!kTiled || G == 4, "tiled weights: one 512-k window per unit");
  constexpr int kWAux = kStream ? 2 : 0;  // buffer-load cache policy of the weight loads (2: nt)
  extern __shared__ u32x4 smem[];
  int pi = 0;
  while (pi + 1 < grp.count && (int)blockIdx.x >= grp.wg_start[pi + 1]) ++pi;
  const uint8_t* __restrict__ codes = grp.p[pi].codes;
  const uint8_t* __restrict__ scales = grp.p[pi].scales;
  const uint16_t* __restrict__ x = grp.p[pi].x;
  float* __restrict__ y = grp.p[pi].y;
  const int n = grp.p[pi].n;
  const int nrb = grp.p[pi].nrb;
  const int brows = grp.p[pi].brows;
  const int y_vec4 = grp.p[pi].y_vec4;
  const float gscale = kNv ? *grp.p[pi].gscale : 1.0f;
  const int ngrid = grp.wg_start[pi + 1] - grp.wg_start[pi];        // this problem's workgroups
  // index among them; mirrored for every second product, so the workgroups holding one
  // row block more than the others are the first ones of product 0 and the last ones of
  // product 1 (the two resident workgroups of a CU, w and w + one grid, then sum to the
  // same number of row blocks)
  const int wgr = (int)blockIdx.x - grp.wg_start[pi];
  const int wg = (pi & 1) ? ngrid - 1 - wgr : wgr;
  const int W = blockDim.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15;  // A row of this lane inside a tile; also its B column
  const int g = lane >> 4;  // which 32-k block of a 128-k group
  const int t0 = blockIdx.y * 16;
  const int mt = min(16, m - t0);
  const int t = t0 + r;
  const bool t_ok = r < mt;
  const int kb = k >> 5;
  const int ngroups = (kb + 3) >> 2;
  // k is walked in `phases` phases of ngroups_p groups (one phase unless the
  // activations of all of k do not fit in LDS); inside a phase wave w owns the
  // groups [gs, gs + nsub·G) of the phase.
  const int gs = wave * G * nsub;  // first group of this wave's slice of a phase
  const uint32_t row_bytes = (uint32_t)(k >> 1);
  // Activations of one phase in LDS, row-major in 16-byte units: row t of the tile
  // starts at unit t·xrs. A row covers every group a wave touches (W·nsub·G >=
  // ngroups_p; the units past the phase or past k hold zeros, so operand reads need
  // no bounds test) plus one unit of padding, which shifts consecutive rows by 16
  // bytes: the 16 lanes of an operand read hit distinct banks.
  const int nq = k >> 3;                   // 16-byte chunks per activation row
  const int nqp = W * nsub * G * 16;       // chunks per padded row of a phase
  const int xrs = nqp + 1;                 // row stride in units
  const int xunits = mt * xrs;
  f32x4* red = reinterpret_cast<f32x4*>(smem + xunits);  // [nred][W][R][64]
  // Lane (r, g) reads chunk grp·16 + 4g + d of row r; rows past m read row 0, which
  // only feeds output columns that are never stored.
  const int xlane = (t_ok ? r : 0) * xrs + 4 * g;

  // this workgroup's work: its row blocks times the phases times the nsub
  // sub-slices of G groups (with several phases a workgroup owns one row block, or
  // in pair mode one pair walked phase-major: all its units form one sequence)
  const int upr = phases * nsub * (kPair ? 2 : 1);  // units per row block (pair)
  const int my_blocks = kPair ? (wg < nrb ? 1 : 0) : (wg < nrb ? (nrb - 1 - wg) / ngrid + 1 : 0);
  const int nunits = my_blocks * upr;
  // unit u -> its row block, phase and sub-slice (j: which block of a pair)
  struct Loc {
    int rb, ph, sub, j;
  };
  auto locate = [&](int u) {
    Loc l;
    const int uu = u % upr;
    l.sub = uu % nsub;
    if constexpr (kPair) {
      l.j = (uu / nsub) & 1;
      l.ph = uu / (2 * nsub);
      l.rb = wg + l.j * ngrid;
    } else {
      l.j = 0;
      l.ph = uu / nsub;
      l.rb = wg + (u / upr) * ngrid;
    }
    return l;
  };

  const uint32_t srow = kNv ? (uint32_t)(k >> 4) : (uint32_t)kb;  // scale bytes per row
  auto load = [&](int u, Block<R, G, kNv>& b) {
    const Loc l = locate(u);
    const int rb = l.rb;
    const int gl0 = gs + l.sub * G;            // first group inside the phase
    const int g0 = l.ph * ngroups_p + gl0;   // first group of k
    // descriptors covering the valid rows of row block rb (none past the last unit;
    // none for the missing second block of a last pair)
    const int row0 = rb * brows;
    const bool live = u < nunits && rb < nrb;
    // lanes of rows past `rows` (the rest of an 8-row block, or past n) read zero
    const int rows = live ? min(brows, n - row0) : 0;
    const int rowc = live ? row0 : 0;
    // tiled (row blocks of 16·R rows): the codes descriptor covers the block's whole
    // 16-row tiles (rows past n are zero there), the scales descriptor the ceil(k/512)
    // windows of the 128-row tile holding the block
    const __amdgpu_buffer_rsrc_t cr =
        kTiled ? make_rsrc(codes + (size_t)rowc * row_bytes, (uint32_t)((rows + 15) & ~15) * row_bytes)
               : make_rsrc(codes + (size_t)rowc * row_bytes, (uint32_t)rows * row_bytes);
    const __amdgpu_buffer_rsrc_t sr =
        kTiled && !kNv ? make_rsrc(scales + (size_t)(rowc >> 7) * (size_t)(ngroups >> 2) * 2048u,
                           rows > 0 ? (uint32_t)(ngroups >> 2) * 2048u : 0u)
               : make_rsrc(scales + (size_t)rowc * srow, (uint32_t)rows * srow);
    // The whole offset goes in voffset (soffset = 0): the range check of a raw
    // buffer load covers voffset + the immediate only.
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int blk = (g0 + j) * 4 + g;
      const bool ok = gl0 + j < ngroups_p && blk < kb;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        // tiled: tile (row tile i, group g0 + j), unit 16g + r
        const uint32_t off = !ok     ? kOutOfRange
                             : kTiled ? (uint32_t)(16 * i) * row_bytes + (uint32_t)(g0 + j) * 1024u + (uint32_t)lane * 16u
                                      : (uint32_t)(16 * i + r) * row_bytes + (uint32_t)blk * 16;
        b.c[i][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(cr, off, 0, kWAux));
      }
    }
#pragma unroll
    for (int q = 0; q < G / 4; ++q) {
      const int grp0 = g0 + 4 * q;
      const bool ok = gl0 + 4 * q < ngroups_p && grp0 < ngroups;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        if constexpr (kTiled && !kNv) {
          // window grp0 / 4, unit = the row's place in its 128-row tile
          const uint32_t off =
              ok ? (uint32_t)(grp0 >> 2) * 2048u + (uint32_t)((rowc & 127) + 16 * i + r) * 16u : kOutOfRange;
          b.s[i][q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, off, 0, kWAux));
        } else if constexpr (kNv) {
          // 8 scale bytes per group: two 16-byte loads for 4 groups
          const uint32_t off = ok ? (uint32_t)(16 * i + r) * srow + (uint32_t)grp0 * 8 : kOutOfRange;
          b.s[i][2 * q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, off, 0, kWAux));
          b.s[i][2 * q + 1] =
              __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, ok ? off + 16u : kOutOfRange, 0, kWAux));
        } else {
          const uint32_t off = ok ? (uint32_t)(16 * i + r) * srow + (uint32_t)grp0 * 4 : kOutOfRange;
          b.s[i][q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, off, 0, kWAux));
        }
      }
    }
  };

  // Activation staging of phase ph by direct global-to-LDS loads. A wave reads only
  // the columns of its own k-slice (units [gs*16, (gs + nsub*G)*16) of every row), so
  // each wave stages exactly those columns and zero-fills their part past the phase's
  // valid chunks: no workgroup barrier between staging and use, at the start or
  // between phases. A wave-load copies 64 consecutive chunks (1 KiB) of one row, so
  // the LDS destination is contiguous as the load-to-LDS form requires (nq, the phase
  // start and the slice start are multiples of 64 chunks).
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + (size_t)t0 * (size_t)k, (uint32_t)(mt * nq) * 16u);
  auto stage = [&](int ph) {
    const int q0 = ph * ngroups_p * 16;                  // first chunk of the phase
    const int nv = min(ngroups_p * 16, nq - q0);         // valid chunks per row
    const int c0 = gs * 16;                              // first chunk of this wave's slice
    const int cw = nsub * G * 16;                        // chunks in the slice
    const int cv = max(0, min(cw, nv - c0));             // valid chunks of the slice
    const int per_row = cv >> 6;
    for (int L = 0; L < mt * per_row; ++L) {
      const int tt = L / per_row;
      const int c = L - tt * per_row;
      __attribute__((address_space(3))) void* dst =
          (__attribute__((address_space(3))) void*)(smem + tt * xrs + c0 + c * 64);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, dst, 16,
                                               (uint32_t)((tt * nq + q0 + c0 + c * 64 + lane) * 16), 0, 0, 0);
    }
    const int zc = cw - cv;
    for (int idx = lane; idx < mt * zc; idx += kWave) {
      const int tt = idx / zc;
      smem[tt * xrs + c0 + cv + (idx - tt * zc)] = u32x4{0u, 0u, 0u, 0u};
    }
  };

  // four accumulator chains per row tile (one per MFMA slice d), so consecutive
  // MFMAs do not wait for each other; summed in a fixed order at the end
  f32x4 acc[R][4];
  f32x4 acc2[kPair ? R : 1][4];  // pair mode: the other row block's accumulators
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int d = 0; d < 4; ++d) acc[i][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (kPair) {
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int d = 0; d < 4; ++d) acc2[i][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  int parity = 0;

  auto compute = [&](int u, const Block<R, G, kNv>& b) {
    const Loc l = locate(u);
    if (phases > 1 && l.ph > 0 && l.sub == 0 && l.j == 0) {
      // first unit of a later phase: this wave restages its own columns (its reads of
      // the previous phase have completed; this also waits for the prefetched unit)
      stage(l.ph);
      __builtin_amdgcn_s_waitcnt(0);
    }
    if constexpr (kPair) {
      // the pair's other row block starts: exchange the accumulator sets
      if (l.sub == 0 && u % upr != 0) {
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const f32x4 tmp = acc[i][d];
            acc[i][d] = acc2[i][d];
            acc2[i][d] = tmp;
          }
      }
    }
    const int gl0 = gs + l.sub * G;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int gl = gl0 + j;
      bf16x8 bb[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) bb[d] = __builtin_bit_cast(bf16x8, smem[xlane + gl * 16 + d]);
      float sf[R], sf2[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        if constexpr (kNv) {
          // this lane's 32 codes are NVFP4 blocks 2g and 2g+1 of group j: scale bytes
          // 8·(j % 4) + 2g and + 1 of the 32 loaded for the group's quadruple
          const int wi = (j % 4) * 2 + g / 2;
          const uint32_t word = b.s[i][(j / 4) * 2 + wi / 4][wi % 4] >> (16 * (g & 1));
          sf[i] = e4m3_to_f32(word & 0xffu);
          sf2[i] = e4m3_to_f32((word >> 8) & 0xffu);
        } else {
          sf[i] = e8m0_to_f32((b.s[i][j / 4][j % 4] >> (8 * g)) & 0xffu);
          sf2[i] = sf[i];
        }
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const bf16x8 a = kNv ? decode8_scaled(b.c[i][j][d], d < 2 ? sf[i] : sf2[i]) : decode8(b.c[i][j][d], sf[i]);
          acc[i][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb[d], acc[i][d], 0, 0, 0);
        }
      }
    }
    if (l.sub != nsub - 1 || l.ph != phases - 1) return;
    // last unit of the row block: sum the waves' partial tiles and store (a missing
    // second block of a pair has rows >= n: nothing is stored)
    const int rb = l.rb;
    f32x4* rp = red + (size_t)(nred == 2 ? parity : 0) * W * R * kWave;
#pragma unroll
    for (int i = 0; i < R; ++i) rp[(wave * R + i) * kWave + lane] = (acc[i][0] + acc[i][1]) + (acc[i][2] + acc[i][3]);
    lds_barrier();
    const int row0 = rb * brows;
    for (int i = wave; i < R; i += W) {
      f32x4 sum = rp[i * kWave + lane];
      for (int w = 1; w < W; ++w) sum += rp[(w * R + i) * kWave + lane];
      if constexpr (kNv) sum *= gscale;
      // lane holds C[4g + e][r]: output row row0 + 16 i + 4 g + e, position t
      const int orow = row0 + 16 * i + 4 * g;
      if (t_ok && 16 * i + 4 * g < brows) {
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
    // one buffer: every wave waits until the sum has read it before the next row
    // block's partial tiles overwrite it
    if (nred == 1) lds_barrier();
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int d = 0; d < 4; ++d) acc[i][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    parity ^= 1;
  };

  // D units in flight: a ring of D register blocks, the loop unrolled by D so every
  // block keeps a fixed role (no register copies, one path into the loop head). The
  // loads of unit u + D go out as soon as unit u has been computed; past the last
  // unit the descriptors have no records and nothing is read. The scheduling
  // barriers keep each prefetch ahead of the next compute's waits.
  Block<R, G, kNv> buf[D];
  stage(0);
#pragma unroll
  for (int i = 0; i < D; ++i) load(i, buf[i]);
  // The direct loads are counted by vmcnt and were issued first: wait for them and the first
  // unit only (the later units' loads, kUnitLoads each, stay in flight while it is computed).
  // No barrier: a wave reads only the columns it staged itself.
  constexpr int kUnitLoads = R * G + R * (kNv ? G / 2 : G / 4);
  static_assert((D - 1) * kUnitLoads < 64, "vmcnt holds at most 63");
  __builtin_amdgcn_s_waitcnt(vmcnt_only((D - 1) * kUnitLoads));
  for (int u = 0; u < nunits; u += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      if (i == 0 || u + i < nunits) compute(u + i, buf[i]);
      load(u + i + D, buf[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ---------------------------------------------------------------------------
// Dense kernel for many activation rows (a batch of sequences × T positions).
//
// With m = 320 the contraction does ~1000 FLOP per weight byte, so the matrix
// cores, not HBM, bound it. A workgroup owns a tile of 128 weight rows × 16·MC
// activation rows and all of k. Its eight waves (two per SIMD) form 2 row halves ×
// 4 k quarters: wave (rh, kq) decodes the weights of rows [64·rh, 64·rh + 64) of
// the tile in registers (4 A operands of 16 rows, loaded straight from HBM, one MX
// block per lane as in the skinny kernel) and multiplies them with the MC B
// operands of every 128-k group g with g % 4 == kq. The activations of each 512-k
// window are staged in LDS by direct global-to-LDS loads, double-buffered, and
// each B operand read feeds 4 MFMAs. The k quarters are summed in LDS at the end
// in a fixed order. Tiles are mapped to XCDs so that the position tiles of one
// weight tile run on the same XCD and share its L2: the weights come from HBM once.
// kTiled: codes in the 1 KiB (16 rows x 128 k) tile layout and scales in the 2 KiB
// (128 rows x 512 k) window layout, so a wave's weight load reads 1 KiB contiguously
// and its scale load of a row tile 256 bytes; the arithmetic is unchanged.
constexpr int kDenseRows = 128;
constexpr int kDenseThreads = 512;

template <int MC, bool kTiled>
__global__ __launch_bounds__(kDenseThreads) void gemm_dense_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ x, float* __restrict__ y, int n, int k, int m, int n_tiles,
    int m_tiles, int y_vec4) {
  constexpr int BM = 16 * MC;
  constexpr int kWaves = kDenseThreads / kWave;
  // Activations of one 512-k window in LDS: row t of the tile holds its 64 chunks of
  // 8 bf16 at units t*64 + (q ^ (t & 15)). A row is 64 consecutive units, so one
  // direct global-to-LDS load (lane L writes unit base + L) stages it; the XOR
  // spreads the 16 rows an operand read touches over distinct banks.
  constexpr int kUnits = BM * 64;
  extern __shared__ u32x4 smem[];
  // workgroup b runs on XCD b % 8; consecutive workgroups of one XCD share a weight tile
  const int xcd = (int)blockIdx.x & 7;
  const int j = (int)blockIdx.x >> 3;
  const int nt = (j / m_tiles) * 8 + xcd;
  const int mtile = j - (j / m_tiles) * m_tiles;
  if (nt >= n_tiles) return;  // uniform for the workgroup, before any barrier

  const int lane = threadIdx.x & (kWave - 1);
  // wave-uniform (a scalar register): the load-to-LDS destination depends on it
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int rh = wave & 1;
  const int kq = wave >> 1;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int kb = k >> 5;
  const int ngroups = kb >> 2;
  // Each wave walks 4 consecutive groups in 4 steps: in step s (block b = s / 4,
  // j = s % 4) wave kq owns group 16b + 4kq + j, and the window staged for the step
  // holds the groups of the 4 k quarters. A wave's 4 groups of a block then have their
  // 16 scale bytes side by side in each row: one 16-byte load per row tile and block
  // instead of a byte load per row tile and step (a per-lane load over 16 rows costs
  // the address unit as much as a code load).
  const int nsteps = 4 * ((ngroups + 15) >> 4);
  auto group_of = [&](int s, int q) { return 16 * (s >> 2) + 4 * q + (s & 3); };
  const uint32_t row_bytes = (uint32_t)(k >> 1);
  const int row0 = nt * kDenseRows;
  const int rows = min(kDenseRows, n - row0);
  // tiled: rows are zero-padded to a multiple of 16, and the tile's scales are its
  // ceil(k/512) windows of 2 KiB
  const int nwin = (ngroups + 3) >> 2;
  const __amdgpu_buffer_rsrc_t cr =
      make_rsrc(codes + (size_t)row0 * row_bytes, (uint32_t)(kTiled ? (rows + 15) & ~15 : rows) * row_bytes);
  const __amdgpu_buffer_rsrc_t sr =
      kTiled ? make_rsrc(scales + (size_t)nt * (size_t)nwin * 2048u, (uint32_t)nwin * 2048u)
             : make_rsrc(scales + (size_t)row0 * kb, (uint32_t)rows * (uint32_t)kb);
  const int t0 = mtile * BM;
  const int mrows = min(BM, m - t0);
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(x + (size_t)t0 * (size_t)k, (uint32_t)mrows * (uint32_t)k * 2u);

  // codes of this wave's 4 row tiles for its group of step s
  struct W4 {
    u32x4 c[4];
  };
  auto load_w = [&](int s, W4& w) {
    const int grp = group_of(s, kq);
    const int blk = grp * 4 + g;
    const bool ok = grp < ngroups;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // tiled: tile (row tile, grp) starts 16 rows' bytes per row tile in, lane L = 16g + r
      const uint32_t rt = (uint32_t)(rh * 64 + 16 * i);
      const uint32_t co = opaque(ok ? (kTiled ? rt * row_bytes + (uint32_t)grp * 1024u + (uint32_t)lane * 16u
                                              : (rt + (uint32_t)r) * row_bytes + (uint32_t)blk * 16)
                                    : kOutOfRange);
      w.c[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(cr, co, 0, 0));
    }
  };
  // scale bytes of this wave's 4 groups of block b, per row tile: byte 4j + g' is block
  // g' of the block's group j. A block past k reads zeros; in a block that k ends
  // inside, the bytes of groups past k are not used (see scale_of).
  auto load_sc = [&](int b, u32x4 (&sc)[4]) {
    const int grp = 16 * b + 4 * kq;
    const bool ok = grp < ngroups;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t row = (uint32_t)(rh * 64 + 16 * i + r);
      // tiled: the 4 groups from grp on are 512-k window grp / 4, whose unit for row is row
      const uint32_t so =
          opaque(ok ? (kTiled ? (uint32_t)(grp >> 2) * 2048u + row * 16u : row * (uint32_t)kb + (uint32_t)grp * 4)
                    : kOutOfRange);
      sc[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, so, 0, 0));
    }
  };
  // Stage the window of step s into buffer buf: wave w stages tile rows w, w + 8, ...;
  // lane L fetches the chunk that belongs at unit 64t + L. Rows past m and groups
  // past k are outside the descriptor and read as zero.
  static_assert(BM % kWaves == 0, "each wave stages the same number of rows");
  auto stage_x_rows = [&](int s, int buf, auto lo, auto hi) {
#pragma unroll
    for (int i = decltype(lo)::value; i < decltype(hi)::value; ++i) {
      const int t = wave + kWaves * i;
      const int q = lane ^ (t & 15);
      // slot q: chunk q % 16 of the group of k quarter q / 16
      const int grp = group_of(s, q >> 4);
      const bool ok = grp < ngroups;
      const uint32_t off =
          opaque(ok ? ((uint32_t)t * (uint32_t)k + (uint32_t)(grp * 128 + (q & 15) * 8)) * 2u : kOutOfRange);
      __attribute__((address_space(3))) void* dst =
          (__attribute__((address_space(3))) void*)(smem + buf * kUnits + 64 * t);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, dst, 16, off, 0, 0, 0);
    }
  };
  auto stage_x = [&](int s, int buf) {
    stage_x_rows(s, buf, std::integral_constant<int, 0>{}, std::integral_constant<int, BM / kWaves>{});
  };
  // the rows of slice d's share when a step's staging is spread over its four MFMA slices
  constexpr int kRowsPer = BM / kWaves;
  auto stage_x_slice = [&](int s, int buf, auto dc) {
    constexpr int d = decltype(dc)::value;
    constexpr int lo = (kRowsPer * d) / 4, hi = (kRowsPer * (d + 1)) / 4;
    stage_x_rows(s, buf, std::integral_constant<int, lo>{}, std::integral_constant<int, hi>{});
  };

  f32x4 acc[4][MC];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < MC; ++c) acc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // block scale of row tile i for step s from the block's scale bytes (1 for a group
  // past k, whose codes read as zero)
  auto scale_of = [&](const u32x4 (&sc)[4], int s, float (&sf)[4]) {
    const bool ok = group_of(s, kq) < ngroups;
#pragma unroll
    for (int i = 0; i < 4; ++i) sf[i] = ok ? e8m0_to_f32((sc[i][s & 3] >> (8 * g)) & 0xffu) : 1.0f;
  };

  auto compute = [&](int buf, const W4& w, const float (&sf)[4], auto&& before_slice) {
    const u32x4* src = smem + buf * kUnits;
    // B operand of slice d, column tile c: lane (r, g) takes chunk kq*16 + 4g + d of
    // tile row 16c + r (the k permutation of the skinny kernel), stored at slot
    // (kq*16 + 4g + d) ^ r of that row. The operands of slice d + 1 are read before
    // the MFMAs of slice d.
    const int xq = (kq * 16 + 4 * g) ^ r;
    const u32x4* bsrc = src + r * 64;
    bf16x8 bb[2][MC];
#pragma unroll
    for (int c = 0; c < MC; ++c) bb[0][c] = __builtin_bit_cast(bf16x8, bsrc[16 * c * 64 + xq]);
    auto slice = [&](auto dc) {
      constexpr int d = decltype(dc)::value;
      before_slice(dc);
      if (d < 3) {
#pragma unroll
        for (int c = 0; c < MC; ++c)
          bb[(d + 1) & 1][c] = __builtin_bit_cast(bf16x8, bsrc[16 * c * 64 + (xq ^ (d + 1))]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 a = decode8(w.c[i][d], sf[i]);
#pragma unroll
        for (int c = 0; c < MC; ++c)
          acc[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb[d & 1][c], acc[i][c], 0, 0, 0);
      }
    };
    slice(std::integral_constant<int, 0>{});
    slice(std::integral_constant<int, 1>{});
    slice(std::integral_constant<int, 2>{});
    slice(std::integral_constant<int, 3>{});
  };

  // The staging and weight loads of step s + 1 are issued before the MFMAs of step
  // s (scheduling barriers keep them there). After the compute each wave waits for
  // its staging loads only (the weight loads issued after them stay in flight; the
  // counter retires in order), then the barrier makes every wave's rows visible.
  W4 wa, wb;
  u32x4 sc[4], scn[4];
  float sf[4];
  load_sc(0, sc);
  stage_x(0, 0);
  load_w(0, wa);
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();
  // Four steps (one block) per iteration and a single exit, so the accumulators keep
  // their registers across the loop; steps past k read only out-of-range (zero)
  // codes and add nothing.
  auto step = [&](int s, auto hc) {
    constexpr int h = decltype(hc)::value;
    if constexpr (kTiled) {
      // the next step's weights first (from HBM: the longest trip), then its activation
      // staging spread over this step's four MFMA slices, so no wave stalls behind a burst
      // of memory instructions it cannot issue
      load_w(s + h + 1, (h & 1) ? wa : wb);
      if constexpr (h == 3) load_sc((s >> 2) + 1, scn);  // the next block's scales, with its first codes
      __builtin_amdgcn_sched_barrier(0);
      scale_of(sc, s + h, sf);
      compute(h & 1, (h & 1) ? wb : wa, sf, [&](auto dc) {
        stage_x_slice(s + h + 1, (h + 1) & 1, dc);
        __builtin_amdgcn_sched_barrier(0);
      });
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);  // the staging was issued last: everything of this step has landed
    } else {
      // row layout (the address arithmetic of its 16-row weight loads leaves no registers for
      // the interleaving): the staging as one burst, then the weights; after the MFMAs wait
      // for the staging only (the weight loads issued after it stay in flight)
      stage_x(s + h + 1, (h + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      load_w(s + h + 1, (h & 1) ? wa : wb);
      if constexpr (h == 3) load_sc((s >> 2) + 1, scn);
      __builtin_amdgcn_sched_barrier(0);
      scale_of(sc, s + h, sf);
      compute(h & 1, (h & 1) ? wb : wa, sf, [](auto) {});
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_only(4 + (h == 3 ? 4 : 0)));  // 4 code loads (+ 4 scale loads)
    }
    lds_barrier();
  };
  for (int s = 0; s < nsteps; s += 4) {
    step(s, std::integral_constant<int, 0>{});
    step(s, std::integral_constant<int, 1>{});
    step(s, std::integral_constant<int, 2>{});
    step(s, std::integral_constant<int, 3>{});
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = scn[i];
  }

  // sum the four k quarters in LDS (the staging buffers are free once every load
  // has landed: the last iteration's loads target windows past k)
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();
  f32x4* red = reinterpret_cast<f32x4*>(smem);  // [3 kq][2 rh][4][MC][64]
  if (kq > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < MC; ++c) red[((((kq - 1) * 2 + rh) * 4 + i) * MC + c) * kWave + lane] = acc[i][c];
  }
  lds_barrier();
  if (kq == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int orow = row0 + rh * 64 + 16 * i + 4 * g;  // lane holds C[4g + e][r]
#pragma unroll
      for (int c = 0; c < MC; ++c) {
        f32x4 sum = acc[i][c];
#pragma unroll
        for (int q = 0; q < 3; ++q) sum += red[(((q * 2 + rh) * 4 + i) * MC + c) * kWave + lane];
        const int tt = t0 + 16 * c + r;
        if (tt < m) {
          float* yp = y + (size_t)tt * (size_t)n + orow;
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
  }
}

// ---------------------------------------------------------------------------
// Fallback when X[mt, k] does not fit in LDS: activations loaded from global
// memory by every wave, one workgroup per row block, waves split k.
template <int R, int S>
struct Stage {
  u32x4 c[R][S];
  uint32_t s[R][S];
  u32x4 xb[S][4];
};

template <int R, int S>
__global__ __launch_bounds__(kMaxWaves * kWave) void gemm_xglobal_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ x, float* __restrict__ y, int n, int k, int m, int gpw,
    int y_vec4) {
  extern __shared__ u32x4 smem[];
  const int W = blockDim.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int row_base = blockIdx.x * (16 * R);
  const int t0 = blockIdx.y * 16;
  const int mt = min(16, m - t0);
  const int t = t0 + r;
  const bool t_ok = r < mt;
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

  f32x4* red = reinterpret_cast<f32x4*>(smem);  // [W][R][64]
#pragma unroll
  for (int i = 0; i < R; ++i) red[(wave * R + i) * kWave + lane] = acc[i];
  __syncthreads();
  for (int i = wave; i < R; i += W) {
    f32x4 sum = red[i * kWave + lane];
    for (int w = 1; w < W; ++w) sum += red[(w * R + i) * kWave + lane];
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

constexpr size_t kMaxLds = 160 * 1024;
constexpr int64_t kDenseMinM = 32;  // above this many activation rows the dense kernel runs
constexpr int kMaxDevices = 64;

// Raise a kernel's dynamic-LDS limit once per device.
template <typename F>
hipError_t allow_lds(F* kernel, std::atomic<bool>* done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < kMaxDevices && done[dev].load(std::memory_order_relaxed)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
  if (e == hipSuccess && dev < kMaxDevices) done[dev].store(true, std::memory_order_relaxed);
  return e;
}

struct Config {
  int R, G;      // row tiles per row block; 128-k groups per unit
  int D;         // units in flight per wave
  int per_cu;    // resident workgroups per CU targeted by the persistent grid
};

inline int y_vec4_ok(const float* y, int64_t n) {
  return (n % 4 == 0) && ((reinterpret_cast<uintptr_t>(y) & 15) == 0);
}

// Waves per workgroup (at most max_waves) and sub-slices per wave for a k of `ngroups`
// 128-k groups.
inline void split_k(int64_t ngroups, int G, int max_waves, int& waves, int& nsub) {
  const int64_t slices = (ngroups + G - 1) / G;  // sub-slices of G groups
  nsub = (int)((slices + max_waves - 1) / max_waves);
  waves = (int)((ngroups + (int64_t)G * nsub - 1) / ((int64_t)G * nsub));
}

// Phase split of k for the main kernel: the fewest phases whose activation tile
// X[mt, k/phases] (padded rows) plus the two reduction buffers fit in LDS. A later
// phase starts on a 4-group (512-k) boundary so its activation rows stay in whole
// 1 KiB windows. Returns false if even 4 groups per phase do not fit.
struct PhasePlan {
  int phases, ngroups_p, waves, nsub, nred;
  size_t lds;
};

// per_cu: resident workgroups per CU the grid is sized for. With one phase, a single
// partial-tile buffer is taken when two would keep that many workgroups from sharing a
// CU's LDS (8 positions over k = 4096: 82 048 bytes with two buffers, 73 856 with one).
inline bool plan_phases(int64_t k, int64_t m, int R, int G, PhasePlan& pp, int per_cu = 1) {
  const int64_t ngroups = (k / 32 + 3) / 4;
  const int64_t mt = m < 16 ? m : 16;
  for (int64_t phases = 1; phases <= ngroups; ++phases) {
    int64_t ngp = (ngroups + phases - 1) / phases;
    if (phases > 1) ngp = (ngp + 3) / 4 * 4;
    if (phases > 1 && (phases - 1) * ngp >= ngroups) continue;  // no empty phase
    // Two resident workgroups per CU (k <= 4096) take four waves of two sub-slices each rather
    // than eight of one: the 8B-class q | k | v 8.38 -> 7.68 µs and gate | up 16.2 -> 15.6 µs at
    // T = 5 (o unchanged); with one workgroup per CU and long k, eight waves stay (down
    // 4096 x 14336: 10.7 µs against 11.9 with four).
    int waves, nsub;
    split_k(ngp, G, per_cu > 1 ? kMaxWaves / 2 : kMaxWaves, waves, nsub);
    const int64_t xrs = (int64_t)waves * nsub * G * 16 + 1;  // padded row stride, 16-byte units
    const size_t xb = (size_t)(mt * xrs) * 16, rb = sizeof(f32x4) * waves * R * kWave;
    if (xb + 2 * rb <= kMaxLds) {
      const bool one = per_cu > 1 && xb + 2 * rb > kMaxLds / per_cu && xb + rb <= kMaxLds / per_cu;
      pp = PhasePlan{(int)phases, (int)ngp, waves, nsub, one ? 1 : 2, xb + (one ? 1 : 2) * rb};
      return true;
    }
    if (ngp <= 4) break;
  }
  return false;
}

template <int R, int G, int D, bool kNv, bool kPair, bool kTiled, bool kStream>
hipError_t launch_main_k(const Config& c, const PhasePlan& pp, const mxs_problem_view* pv, int count,
                         int64_t k, int64_t m, hipStream_t stream) {
  static std::atomic<bool> done[kMaxDevices];
  hipError_t e = allow_lds(&gemm_skinny_kernel<R, G, D, kNv, kPair, kTiled, kStream>, done);
  if (e != hipSuccess) return e;
  Group grp{};
  grp.count = count;
  const int64_t budget = (int64_t)device_cus() * c.per_cu;
  // Persistent grid split between the products: in proportion to their row blocks, at
  // least one workgroup each, never more than a product's row blocks, and never more
  // than the budget in total (one workgroup past it would run as a second round: the
  // 70B-class q | k | v took 21.9 µs with 257 workgroups). Spare workgroups go to the
  // product with the most row blocks per workgroup. With several phases every row block
  // (or pair of row blocks) gets its own workgroup.
  int64_t share[kMaxGroup];
  int64_t nrbs[kMaxGroup];
  int brows[kMaxGroup];
  // 8-row blocks for every product but the largest when the group's 16-row blocks leave
  // resident slots unused and the halves still fit: q | k | v of the 8B-class layer is
  // 256 + 64 + 64 blocks on 512 slots (two per CU), so half the CUs held two blocks and
  // half one; with k and v in 8-row blocks every CU holds one q block and one half block.
  // Tiled weights keep 16-row blocks: a half block would read 128-byte pieces of each tile,
  // and q | k | v measured as fast or faster without halves there (8.3 vs 8.5 µs at T = 1,
  // 9.5 vs 9.8 at T = 8).
  int big = 0;
  int64_t nrb16 = 0, half_total = 0;
  for (int i = 0; i < count; ++i) {
    nrb16 += (pv[i].n + 16 * R - 1) / (16 * R);
    if (pv[i].n > pv[big].n) big = i;
  }
  for (int i = 0; i < count; ++i) half_total += i == big ? (pv[i].n + 15) / 16 : (pv[i].n + 7) / 8;
  const bool halves = !kTiled && R == 1 && pp.phases == 1 && count > 1 && nrb16 < budget && half_total <= budget;
  for (int i = 0; i < count; ++i) brows[i] = halves && i != big ? 8 : 16 * R;
  int64_t sum = 0, total_rb = 0;
  for (int i = 0; i < count; ++i) {
    nrbs[i] = (pv[i].n + brows[i] - 1) / brows[i];
    total_rb += nrbs[i];
  }
  for (int i = 0; i < count; ++i) {
    int64_t sh = pp.phases > 1 ? (kPair ? (nrbs[i] + 1) / 2 : nrbs[i]) : budget * nrbs[i] / total_rb;
    sh = sh > nrbs[i] ? nrbs[i] : sh;
    share[i] = sh < 1 ? 1 : sh;
    sum += share[i];
  }
  if (pp.phases == 1) {
    while (sum > budget) {  // only when the minimum of one per product overshoots
      int top = 0;
      for (int i = 1; i < count; ++i)
        if (share[i] > share[top]) top = i;
      if (share[top] <= 1) break;
      --share[top];
      --sum;
    }
    while (sum < budget) {
      int best = -1;
      int64_t best_load = 0;
      for (int i = 0; i < count; ++i) {
        if (share[i] >= nrbs[i]) continue;
        const int64_t load = (nrbs[i] + share[i] - 1) / share[i];
        if (load > best_load) {
          best_load = load;
          best = i;
        }
      }
      if (best < 0) break;
      ++share[best];
      ++sum;
    }
  }
  int start = 0;
  for (int i = 0; i < count; ++i) {
    const int64_t nrb = nrbs[i];
    grp.p[i] = Problem{pv[i].codes, pv[i].scales, pv[i].x, pv[i].y, kNv ? pv[i].gscale : nullptr, (int)pv[i].n, (int)nrb,
                       y_vec4_ok(pv[i].y, pv[i].n), brows[i]};
    grp.wg_start[i] = start;
    start += (int)share[i];
  }
  grp.wg_start[count] = start;
  gemm_skinny_kernel<R, G, D, kNv, kPair, kTiled, kStream><<<dim3((unsigned)start, (unsigned)((m + 15) / 16)),
                                                            dim3(pp.waves * kWave), pp.lds, stream>>>(
      grp, (int)k, (int)m, pp.nsub, pp.phases, pp.ngroups_p, pp.nred);
  return hipGetLastError();
}

// Non-temporal weight loads when one position tile reads every weight once (m <= 16).
template <int R, int G, int D, bool kNv = false, bool kPair = false, bool kTiled = false>
hipError_t launch_main(const Config& c, const PhasePlan& pp, const mxs_problem_view* pv, int count,
                       int64_t k, int64_t m, hipStream_t stream) {
  if (m <= 16) return launch_main_k<R, G, D, kNv, kPair, kTiled, true>(c, pp, pv, count, k, m, stream);
  return launch_main_k<R, G, D, kNv, kPair, kTiled, false>(c, pp, pv, count, k, m, stream);
}

template <int R, int S>
hipError_t launch_xglobal(int gpw, const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                          const uint16_t* x, int64_t m, float* y, hipStream_t stream) {
  const int ngroups = (int)((k / 32 + 3) / 4);
  int waves = (ngroups + gpw - 1) / gpw;
  if (waves > kMaxWaves) {
    gpw = (ngroups + kMaxWaves - 1) / kMaxWaves;
    waves = (ngroups + gpw - 1) / gpw;
  }
  const size_t lds = sizeof(f32x4) * (size_t)waves * R * kWave;
  dim3 grid((unsigned)((n + 16 * R - 1) / (16 * R)), (unsigned)((m + 15) / 16));
  gemm_xglobal_kernel<R, S><<<grid, dim3(waves * kWave), lds, stream>>>(
      codes, scales, x, y, (int)n, (int)k, (int)m, gpw, y_vec4_ok(y, n));
  return hipGetLastError();
}

// Dense kernel: 16·MC activation rows per tile.
constexpr int kDenseMC = 5;

inline bool dense_ok(int64_t k, int64_t m) {
  return m > kDenseMinM && k % 128 == 0 && k <= (int64_t(1) << 23);
}

// the dense grid's thread count must fit 32 bits (n beyond ~1M rows at m = 65536)
inline bool dense_grid_ok(int64_t n, int64_t m) {
  const int64_t wgs = (n + 8 * kDenseRows - 1) / (8 * kDenseRows) * 8 * ((m + 16 * kDenseMC - 1) / (16 * kDenseMC));
  return wgs <= (int64_t)0xffffffffu / kDenseThreads;
}

template <bool kTiled>
hipError_t launch_dense(const mxs_problem_view& p, int64_t k, int64_t m, hipStream_t stream) {
  constexpr int MC = kDenseMC;
  static std::atomic<bool> done[kMaxDevices];
  hipError_t e = allow_lds(&gemm_dense_kernel<MC, kTiled>, done);
  if (e != hipSuccess) return e;
  const int n_tiles = (int)((p.n + kDenseRows - 1) / kDenseRows);
  const int m_tiles = (int)((m + 16 * MC - 1) / (16 * MC));
  const int64_t wgs = (int64_t)((n_tiles + 7) / 8) * 8 * m_tiles;
  if (!dense_grid_ok(p.n, m)) return hipErrorInvalidConfiguration;
  const size_t lds = 2 * sizeof(u32x4) * (16 * MC * 64);
  gemm_dense_kernel<MC, kTiled><<<dim3((unsigned)wgs), dim3(kDenseThreads), lds, stream>>>(
      p.codes, p.scales, p.x, p.y, (int)p.n, (int)k, (int)m, n_tiles, m_tiles, y_vec4_ok(p.y, p.n));
  return hipGetLastError();
}

// One launch for up to kMaxGroup problems with the same k and m (persistent kernel), or
// one dense or fallback launch per problem.
hipError_t launch_group(Config c, const mxs_problem_view* pv, int count, int64_t k, int64_t m,
                        hipStream_t stream) {
  bool dense = dense_ok(k, m);
  for (int i = 0; i < count; ++i) dense = dense && dense_grid_ok(pv[i].n, m);
  if (dense) {
    for (int i = 0; i < count; ++i) {
      const hipError_t e = launch_dense<false>(pv[i], k, m, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // Main kernel: 16-byte scale loads need k % 512 == 0 and 16-byte aligned scales; a row
  // block's bytes (64 rows at most) must fit a 32-bit buffer range.
  bool aligned = (k % 512 == 0) && k <= (int64_t(1) << 24);
  for (int i = 0; i < count; ++i)
    aligned = aligned && ((reinterpret_cast<uintptr_t>(pv[i].scales) & 15) == 0);
  PhasePlan pp;
  if (aligned && plan_phases(k, m, c.R, c.G, pp, c.per_cu)) {
    // With several phases a workgroup walks a pair of 16-row blocks phase by phase
    // (kPair) when the pairs still give every CU a workgroup (8192 x 28672 at T = 5:
    // 39.2 -> 33.2 µs); with fewer row blocks (4096 x 14336 at T = 8: 128 pairs,
    // 13.0 -> 17.7 µs) each row block keeps its own workgroup. Two row tiles per
    // block (R = 2) measured slower than either: 42.9 µs for 8192 x 28672.
    int64_t pairs = 0;
    for (int i = 0; i < count; ++i) pairs += ((pv[i].n + 15) / 16 + 1) / 2;
    if (pp.phases > 1 && pairs >= device_cus() && c.R == 1 && c.G == 4 && c.D == 2)
      return launch_main<1, 4, 2, false, true>(c, pp, pv, count, k, m, stream);
    if (c.R == 1 && c.G == 4 && c.D == 2) return launch_main<1, 4, 2>(c, pp, pv, count, k, m, stream);
    return hipErrorInvalidValue;  // choose() returns the one configuration built
  }
  for (int i = 0; i < count; ++i) {
    const hipError_t e =
        launch_xglobal<2, 4>(4, pv[i].codes, pv[i].scales, pv[i].n, k, pv[i].x, m, pv[i].y, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Tiled codes and scales (launch_tile_codes / launch_tile_scales): the skinny kernel (one
// 16-row tile per row block, 4 groups per unit, so a unit is one 512-k window) for m <= 32
// with k % 512 == 0, with the same pair rule as the row layout; else the dense kernel per
// product.
hipError_t launch_group_tiled(Config c, const mxs_problem_view* pv, int count, int64_t k, int64_t m,
                              hipStream_t stream) {
  PhasePlan pp;
  const bool skinny = m <= kDenseMinM && k % 512 == 0 && k <= (int64_t(1) << 24) &&
                      plan_phases(k, m, 1, 4, pp, c.per_cu) && pp.ngroups_p % 4 == 0;
  if (!skinny) {
    for (int i = 0; i < count; ++i) {
      const hipError_t e = launch_dense<true>(pv[i], k, m, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const Config c1{1, 4, 2, c.per_cu};
  int64_t pairs = 0;
  for (int i = 0; i < count; ++i) pairs += ((pv[i].n + 15) / 16 + 1) / 2;
  if (pp.phases > 1 && pairs >= device_cus()) return launch_main<1, 4, 2, false, true, true>(c1, pp, pv, count, k, m, stream);
  return launch_main<1, 4, 2, false, false, true>(c1, pp, pv, count, k, m, stream);
}

hipError_t launch_cfg(Config c, const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                      const uint16_t* x, int64_t m, float* y, hipStream_t stream) {
  const mxs_problem_view pv{codes, scales, x, y, n};
  return launch_group(c, &pv, 1, k, m, stream);
}

// Tile choice from sweeps of (R, G, units in flight, workgroups per CU) over the 8B-
// and 70B-class shapes at T = 5 and 8: one 16-row tile per row block, 4 groups per
// unit and two units in flight won or tied everywhere (four units in flight was
// 5-30% slower); two resident workgroups per CU for k <= 4096, one above.
Config choose(int64_t n, int64_t k) {
  (void)n;
  return Config{1, 4, 2, k <= 4096 ? 2 : 1};
}

}  // namespace

// Compute units of the current device (256 on MI355X), read once per device: the persistent
// grids are sized as resident workgroups per CU times this count.
int device_cus() {
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int c = cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
  if (dev < kMaxDevices) cus[dev].store(c, std::memory_order_relaxed);
  return c;
}

hipError_t launch_verify_gemm(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                              const uint16_t* x, int64_t m, float* y, hipStream_t stream) {
  return launch_cfg(choose(n, k), codes, scales, n, k, x, m, y, stream);
}

hipError_t launch_verify_gemm_tiled(const uint8_t* tiled_codes, const uint8_t* tiled_scales, int64_t n, int64_t k,
                                    const uint16_t* x, int64_t m, float* y, hipStream_t stream) {
  const mxs_problem_view pv{tiled_codes, tiled_scales, x, y, n};
  return launch_group_tiled(choose(n, k), &pv, 1, k, m, stream);
}

hipError_t launch_verify_gemm_grouped_tiled(const mxs_problem_view* pv, int count, int64_t k, int64_t m,
                                            hipStream_t stream) {
  int64_t n_total = 0;
  for (int i = 0; i < count; ++i) n_total += pv[i].n;
  for (int i0 = 0; i0 < count; i0 += kMaxGroup) {
    const int cnt = count - i0 < kMaxGroup ? count - i0 : kMaxGroup;
    const hipError_t e = launch_group_tiled(choose(n_total, k), pv + i0, cnt, k, m, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// NVFP4 weights: the skinny kernel for every m (a 16-position tile per grid row), k % 512 == 0
// and 16-byte aligned scales checked by the caller; up to kMaxGroup products per launch.
// kTiled: codes in the tiled layout of launch_tile_codes, scales in the row layout.
template <bool kTiled = false>
static hipError_t launch_nvfp4_group(const mxs_problem_view* pv, int count, int64_t k, int64_t m,
                                     hipStream_t stream) {
  int64_t n_total = 0, nrb2 = 0;
  for (int i = 0; i < count; ++i) {
    n_total += pv[i].n;
    nrb2 += (pv[i].n + 31) / 32;
  }
  const Config c = choose(n_total, k);
  PhasePlan pp;
  if (!plan_phases(k, m < 16 ? m : 16, c.R, c.G, pp, c.per_cu)) return hipErrorInvalidValue;
  if (pp.phases > 1) {
    // with several phases a workgroup owns one row block: two row tiles per block when
    // that still leaves a workgroup per CU
    PhasePlan pp2;
    if (nrb2 >= device_cus() && plan_phases(k, m < 16 ? m : 16, 2, c.G, pp2))
      return launch_main<2, 4, 2, true, false, kTiled>(Config{2, c.G, c.D, c.per_cu}, pp2, pv, count, k, m, stream);
  }
  return launch_main<1, 4, 2, true, false, kTiled>(c, pp, pv, count, k, m, stream);
}

hipError_t launch_nvfp4_verify_gemm(const uint8_t* codes, const uint8_t* scales, const float* gscale,
                                    int64_t n, int64_t k, const uint16_t* x, int64_t m, float* y,
                                    hipStream_t stream) {
  mxs_problem_view pv{codes, scales, x, y, n};
  pv.gscale = gscale;
  return launch_nvfp4_group(&pv, 1, k, m, stream);
}

hipError_t launch_nvfp4_verify_gemm_grouped(const mxs_problem_view* pv, int count, int64_t k, int64_t m,
                                            hipStream_t stream) {
  for (int i0 = 0; i0 < count; i0 += kMaxGroup) {
    const int cnt = count - i0 < kMaxGroup ? count - i0 : kMaxGroup;
    const hipError_t e = launch_nvfp4_group(pv + i0, cnt, k, m, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_nvfp4_verify_gemm_grouped_tiled(const mxs_problem_view* pv, int count, int64_t k, int64_t m,
                                                  hipStream_t stream) {
  for (int i0 = 0; i0 < count; i0 += kMaxGroup) {
    const int cnt = count - i0 < kMaxGroup ? count - i0 : kMaxGroup;
    const hipError_t e = launch_nvfp4_group<true>(pv + i0, cnt, k, m, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_verify_gemm_grouped(const mxs_problem_view* pv, int count, int64_t k, int64_t m,
                                      hipStream_t stream) {
  int64_t n_total = 0;
  for (int i = 0; i < count; ++i) n_total += pv[i].n;
  for (int i0 = 0; i0 < count; i0 += kMaxGroup) {
    const int cnt = count - i0 < kMaxGroup ? count - i0 : kMaxGroup;
    const hipError_t e = launch_group(choose(n_total, k), pv + i0, cnt, k, m, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}


}  // namespace mxs
