// mx_verify_gemm_act: Y[m, n] = X^[m, k] · Ŵ[n, k]ᵀ with MX-FP4 weights and MX-quantized
// activations (MX-FP8 E4M3 or MX-FP4 E2M1, an E8M0 scale per 32 values): the W4A8 /
// W4A4 forms of the verify GEMM ("Module 11. Speculative Decoding and Quantization"
// §11 and §12), for the batched verification of many sequences.
//
// The block-scaled matrix instruction v_mfma_scale_f32_16x16x128_f8f6f4 takes both
// operands in their stored formats with one E8M0 scale byte per lane, so nothing is
// decoded: a lane's A operand is the 16 code bytes of one 32-weight MX block (the
// same load as the weight-only kernels) and its scale byte; its B operand is one
// 32-value activation block of one position with that block's scale. Lane (r, g)
// covers k-block g of the 128-k group: FP4 operands hold the block's 32 values in
// order; an 8-bit operand holds values 16·h .. 16·h + 15 of blocks g' = g/2 and
// g/2 + 2 (bytes 0-15 and 16-31) for h = g % 2, while the lane's scale still belongs
// to block g. A and B therefore keep the natural k order of the group.
//
// Work split as in the weight-only dense kernel: a workgroup owns 128 weight rows × 80
// positions and all of k; 8 waves = 2 row halves × 4 k quarters; weights go from
// HBM straight into registers; the activation codes of each 512-k window are staged
// in LDS by direct global-to-LDS loads into an XOR-swizzled tile, double-buffered;
// each B operand read feeds 4 MFMAs; the k quarters are summed in LDS in a fixed
// order; position tiles of one weight tile share an XCD's L2.
#include "common.hpp"
#include "internal.hpp"

namespace mxs {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kRows = 128;  // weight rows per workgroup tile
constexpr int kMC = 5;      // 16-position column tiles per workgroup tile
constexpr int kRQ = 2;      // row groups per tile: 4·kRQ waves, 8/kRQ row tiles per wave

// kTiled: the weight codes come in the tiled layout of mxfp4_tile_codes (one 1 KiB tile
// per 16 rows x 128-k group, the lanes of an operand load in order), so each wave-wide
// operand load reads 1 KiB contiguously instead of 64 bytes from each of 16 rows; the
// weight scales in the layout of mxfp4_tile_scales (2 KiB per 128 rows x 512-k window),
// staged by two 1 KiB loads per window instead of eight loads of 16 rows x 16 bytes.
template <int MC, int AF, int RQ, bool kTiled = false>
__global__ __launch_bounds__(256 * RQ) void gemm_act_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const uint8_t* __restrict__ acodes, const uint8_t* __restrict__ ascales, float* __restrict__ y,
    int n, int k, int m, int n_tiles, int m_tiles, int y_vec4) {
  constexpr int BM = 16 * MC;
  constexpr int kWaves = 4 * RQ;  // RQ row groups × 4 k quarters
  constexpr int RT = 8 / RQ;      // 16-row tiles per wave
  // 16-byte units per position in one 512-k window: 32 (8-bit codes) or 16 (4-bit)
  constexpr int kRowUnits = AF == MXS_ACT_FP8 ? 32 : 16;
  constexpr int kRowsPerLoad = kWave / kRowUnits;  // positions one wave-wide code load covers
  constexpr int kLoads = BM / kRowsPerLoad;        // wave-wide code loads per window
  constexpr int kUnits = BM * kRowUnits;           // code units per staging buffer
  // A staging buffer holds the window's activation codes, then its scale dwords (one
  // 16-byte unit of 4 groups per weight row, then one per position), then a 1 KiB pad.
  // Scales go through LDS like the codes: loaded per lane from global memory they cost
  // as many address cycles as the codes (16 rows per instruction) for 1/16 the bytes.
  constexpr int kScaleLoads = (kRows + BM) / 16;   // 4-byte-per-lane loads: 16 rows each
  constexpr int kPerWave = (kLoads + kWaves - 1) / kWaves;
  constexpr int kWsc = kUnits;              // first weight-scale unit
  constexpr int kXsc = kUnits + kRows;      // first activation-scale unit
  constexpr int kPadU = kUnits + kRows + BM;
  constexpr int kBufU = kPadU + kWave;
  // The two staging buffers are separate LDS objects, so the compiler can tell that
  // the direct loads into one never alias the operand reads of the other and does not
  // make those reads wait for the loads just issued. Surplus wave-wide loads (when the
  // loads of a window do not divide evenly among the waves) read nothing into the pad:
  // every wave issues the same loads without a branch, so wait counts stay exact.
  __shared__ u32x4 xbuf0[kBufU];
  __shared__ u32x4 xbuf1[kBufU];
  __shared__ u32x4 xbuf2[kBufU];
  // workgroup b runs on XCD b % 8; consecutive workgroups of one XCD share a weight tile
  const int xcd = (int)blockIdx.x & 7;
  const int j = (int)blockIdx.x >> 3;
  const int nt = (j / m_tiles) * 8 + xcd;
  const int mtile = j - (j / m_tiles) * m_tiles;
  if (nt >= n_tiles) return;  // uniform for the workgroup, before any barrier

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int rq = wave % RQ;
  const int kq = wave / RQ;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int kb = k >> 5;
  const int ngroups = kb >> 2;
  const int nsteps = (ngroups + 3) >> 2;  // 512-k windows
  // Each weight tile walks the windows starting at its own offset, so the tiles do not
  // all read the same column of the matrix at once.
  const int s0 = (int)(((unsigned)nt * 13u) % (unsigned)max(nsteps, 1));
  auto window = [&](int s) { return s < nsteps ? (s + s0 < nsteps ? s + s0 : s + s0 - nsteps) : s; };
  const uint32_t row_bytes = (uint32_t)(k >> 1);
  const uint32_t arow_bytes = AF == MXS_ACT_FP8 ? (uint32_t)k : (uint32_t)(k >> 1);
  const int row0 = nt * kRows;
  const int rows = min(kRows, n - row0);
  // a tiled matrix holds whole 16-row tiles (rows past n are zero); both layouts put
  // row0 at byte row0 * row_bytes
  const int crows = kTiled ? min(kRows, ((n + 15) & ~15) - row0) : rows;
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(codes + (size_t)row0 * row_bytes, (uint32_t)crows * row_bytes);
  // tiled scales: this tile's windows, 2 KiB each, at (nt * windows + window) * 2 KiB
  const __amdgpu_buffer_rsrc_t sr =
      kTiled ? make_rsrc(scales + (size_t)nt * (size_t)nsteps * 2048u, (uint32_t)nsteps * 2048u)
             : make_rsrc(scales + (size_t)row0 * kb, (uint32_t)rows * (uint32_t)kb);
  const int t0 = mtile * BM;
  const int mrows = min(BM, m - t0);
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(acodes + (size_t)t0 * arow_bytes, (uint32_t)mrows * arow_bytes);
  const __amdgpu_buffer_rsrc_t xsr = make_rsrc(ascales + (size_t)t0 * kb, (uint32_t)mrows * (uint32_t)kb);

  // (load offsets pass through opaque(): see common.hpp)
  // the codes of this wave's RT row tiles for its group of step s (rows past n read 0)
  struct Ops {
    u32x4 c[RT];
  };
  auto load_ops = [&](int s, Ops& o) {
    const int grp = 4 * window(s) + kq;
    const int blk = grp * 4 + g;
    const bool ok = grp < ngroups;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const uint32_t row = (uint32_t)(rq * 16 * RT + 16 * i + r);
      // tiled: tile (row tile, group) is 1 KiB at ((row tile) * groups + group) * 1 KiB,
      // and lane (r, g) holds the 16 bytes of row r, block g
      const uint32_t tile = (uint32_t)(rq * RT + i) * (uint32_t)ngroups + (uint32_t)grp;
      const uint32_t co = opaque(ok ? (kTiled ? tile * 1024u + (uint32_t)lane * 16u : row * row_bytes + (uint32_t)blk * 16)
                                    : kOutOfRange);
      o.c[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(cr, co, 0, 0));
    }
  };
  constexpr int kOpLoads = RT;  // VMEM loads of one load_ops

  // Stage window s into buffer buf. Codes: unit u of position t sits at t·kRowUnits + u
  // and holds chunk q = u ^ (t mod 16) of the window; one wave-wide load L writes the
  // kRowsPerLoad positions kRowsPerLoad·L.. contiguously. Scales: scale load J writes
  // 16 rows (weight rows for J < kRows/16, then positions) × 4 dwords, dword d of a row
  // being group 4·window + d. Positions past m, rows past n and groups past k are
  // outside the descriptors or masked and read as zero.
  auto stage_x = [&](int sl, u32x4* buf) {
    const int s = window(sl);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int L = wave + kWaves * i;
      const bool live = kLoads % kWaves == 0 || L < kLoads;  // wave-uniform
      const int t = L * kRowsPerLoad + lane / kRowUnits;
      const int u = lane % kRowUnits;
      const int q = u ^ (t & 15);
      const int qg = AF == MXS_ACT_FP8 ? q >> 3 : q >> 2;  // group of the chunk inside the window
      const bool ok = live && 4 * s + qg < ngroups;
      const uint32_t off = ok ? (uint32_t)t * arow_bytes + (uint32_t)(s * kRowUnits + q) * 16u : kOutOfRange;
      __attribute__((address_space(3))) void* dst =
          (__attribute__((address_space(3))) void*)(buf + (live ? kWave * L : kPadU));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, dst, 16, off, 0, 0, 0);
    }
    if constexpr (kTiled) {
      // weight scales: waves 0 and 1 each copy 1 KiB of the window's 2 KiB (rows 64w ..
      // 64w + 63); the other waves issue the same load into the pad, reading nothing
      const bool live = wave < 2;
      const uint32_t off = live && s < nsteps ? (uint32_t)s * 2048u + (uint32_t)wave * 1024u + (uint32_t)lane * 16u
                                              : kOutOfRange;
      __attribute__((address_space(3))) void* dst =
          (__attribute__((address_space(3))) void*)(buf + (live ? kWsc + 64 * wave : kPadU));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, dst, 16, off, 0, 0, 0);
    }
    // the remaining 4-byte-per-lane scale loads: weight rows (row layout only), then positions
    constexpr int kJ0 = kTiled ? kRows / 16 : 0;
    constexpr int kJPerWave = (kScaleLoads - kJ0 + kWaves - 1) / kWaves;
#pragma unroll
    for (int i = 0; i < kJPerWave; ++i) {
      const int J = kJ0 + wave + kWaves * i;  // wave-uniform
      const bool wsc = J < kRows / 16;
      const bool live = J < kScaleLoads;
      const int row = (wsc ? J : J - kRows / 16) * 16 + lane / 4;
      const int d = lane & 3;
      const bool ok = live && 4 * s + d < ngroups;
      const uint32_t off = ok ? (uint32_t)row * (uint32_t)kb + (uint32_t)(16 * s + 4 * d) : kOutOfRange;
      __attribute__((address_space(3))) void* dst =
          (__attribute__((address_space(3))) void*)(buf + (live ? kWsc + 16 * J : kPadU));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wsc ? sr : xsr, dst, 4, off, 0, 0, 0);
    }
  };

  f32x4 acc[RT][MC];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int c = 0; c < MC; ++c) acc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const u32x4* src, const Ops& o) {
    // scale byte of block g of group kq: byte 4·kq + g of the row's scale unit
    const uint8_t* sb = reinterpret_cast<const uint8_t*>(src);
    uint32_t sw[RT], sx[MC];
#pragma unroll
    for (int i = 0; i < RT; ++i) sw[i] = sb[(kWsc + rq * 16 * RT + 16 * i + r) * 16 + 4 * kq + g];
#pragma unroll
    for (int c = 0; c < MC; ++c) sx[c] = sb[(kXsc + 16 * c + r) * 16 + 4 * kq + g];
    i32x8 a[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i)
      a[i] = i32x8{(int)o.c[i][0], (int)o.c[i][1], (int)o.c[i][2], (int)o.c[i][3], 0, 0, 0, 0};
    // one column tile at a time: its B operand, read from LDS while the previous tile's
    // MFMAs run, feeds RT MFMAs
    auto read_b = [&](int c) {
      const int t = 16 * c + r;  // t mod 16 == r
      if constexpr (AF == MXS_ACT_FP8) {
        // values 16h .. 16h+15 of blocks g/2 and g/2 + 2 of group kq: chunks 8kq + g, 8kq + g + 4
        const u32x4 lo = src[t * kRowUnits + ((8 * kq + g) ^ r)];
        const u32x4 hi = src[t * kRowUnits + ((8 * kq + g + 4) ^ r)];
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      } else {
        const u32x4 v = src[t * kRowUnits + ((4 * kq + g) ^ r)];  // block g of group kq
        return i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
      }
    };
    i32x8 bb[2];
    bb[0] = read_b(0);
#pragma unroll
    for (int c = 0; c < MC; ++c) {
      if (c + 1 < MC) bb[(c + 1) & 1] = read_b(c + 1);
#pragma unroll
      for (int i = 0; i < RT; ++i)
        acc[i][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], bb[c & 1], acc[i][c], MXS_ACT_FP4, AF, 0,
                                                                     (int)sw[i], 0, (int)sx[c]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The accumulators pass through an empty asm after each step's MFMAs: the MFMAs are
  // pure, and without it the compiler sinks them below the next step's loads, where
  // their operands' wait counts then cover those loads too.
  auto pin_acc = [&]() {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int c = 0; c < MC; ++c) asm volatile("" : "+v"(acc[i][c]));
  };

  // Staging and operand loads of step s + 2 go out before the MFMAs of step s, the staging
  // first: the counter retires in order, so at the end of step s each wave waits for the
  // staging of step s + 1 (issued a step before) while the operands of step s + 1 (issued
  // after it) and everything of step s + 2 stay in flight; then the barrier makes every
  // wave's positions visible. Three staging buffers and three operand sets rotate.
  constexpr int kStageLoads = kPerWave + (kTiled ? 1 : 0) + ((kScaleLoads - (kTiled ? kRows / 16 : 0) + kWaves - 1) / kWaves);
  Ops o0, o1, o2;
  stage_x(0, xbuf0);
  load_ops(0, o0);
  stage_x(1, xbuf1);
  load_ops(1, o1);
  __builtin_amdgcn_s_waitcnt(vmcnt_only(kStageLoads + kOpLoads));
  lds_barrier();
  // The step barrier carries no LDS release fence: such a fence also waits for every direct
  // global-to-LDS load in flight (they write LDS), which would drain the staging of step
  // s + 2. Each wave has waited for its own staging of step s + 1 and read its operands of
  // step s (the MFMAs consumed them), and LDS needs no cache maintenance inside a CU, so a
  // bare barrier (with a compiler memory clobber) orders the steps.
  auto step_barrier = []() { asm volatile("s_barrier" ::: "memory"); };
  auto step = [&](int sc, u32x4* cur, const Ops& oc, u32x4* nxt, Ops& on) {
    stage_x(sc + 2, nxt);
    __builtin_amdgcn_sched_barrier(0);
    load_ops(sc + 2, on);
    __builtin_amdgcn_sched_barrier(0);
    if (sc < nsteps) compute(cur, oc);  // uniform: past the last window the step adds nothing
    pin_acc();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * kOpLoads + kStageLoads));
    step_barrier();
  };
  for (int s = 0; s < nsteps; s += 3) {
    step(s, xbuf0, o0, xbuf2, o2);
    step(s + 1, xbuf1, o1, xbuf0, o0);
    step(s + 2, xbuf2, o2, xbuf1, o1);
  }

  // Sum the four k quarters through the staging buffers (free once every load has
  // landed: the last iteration's loads target windows past k), one quarter at a time,
  // the first half of the row groups in one buffer and the second half in the other;
  // k quarter 0 adds them in the order 1, 2, 3 and stores.
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();
  constexpr int kTileRegs = RT * MC * kWave;  // f32x4 partial tiles of one wave
  static_assert(sizeof(xbuf0) >= sizeof(f32x4) * (RQ / 2) * kTileRegs, "half the row groups fit a buffer");
  f32x4* red = reinterpret_cast<f32x4*>(rq < RQ / 2 ? xbuf0 : xbuf1) + (rq % (RQ / 2)) * kTileRegs;
  for (int q = 1; q < 4; ++q) {
    if (kq == q) {
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int c = 0; c < MC; ++c) red[(i * MC + c) * kWave + lane] = acc[i][c];
    }
    lds_barrier();
    if (kq == 0) {
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int c = 0; c < MC; ++c) acc[i][c] += red[(i * MC + c) * kWave + lane];
    }
    lds_barrier();
  }
  if (kq == 0) {
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int orow = row0 + rq * 16 * RT + 16 * i + 4 * g;  // lane holds C[4g + e][r]
#pragma unroll
      for (int c = 0; c < MC; ++c) {
        const f32x4 sum = acc[i][c];
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

template <int AF, bool kTiled>
hipError_t launch(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k, const uint8_t* acodes,
                  const uint8_t* ascales, int64_t m, float* y, hipStream_t stream) {
  const int n_tiles = (int)((n + kRows - 1) / kRows);
  const int m_tiles = (int)((m + 16 * kMC - 1) / (16 * kMC));
  const int64_t wgs = (int64_t)((n_tiles + 7) / 8) * 8 * m_tiles;
  const int y_vec4 = (n % 4 == 0) && ((reinterpret_cast<uintptr_t>(y) & 15) == 0);
  gemm_act_kernel<kMC, AF, kRQ, kTiled><<<dim3((unsigned)wgs), dim3(256 * kRQ), 0, stream>>>(
      codes, scales, acodes, ascales, y, (int)n, (int)k, (int)m, n_tiles, m_tiles, y_vec4);
  return hipGetLastError();
}

// Row-layout codes [n, k/2] -> tiled codes: unit (16 bytes) u of the output, with
// u = (row tile * groups + group) * 64 + 16 * g + r, is row 16 * tile + r, MX block
// 4 * group + g of the input; rows past n are zero. One thread per unit.
__global__ __launch_bounds__(256) void tile_codes_kernel(const uint8_t* __restrict__ codes, int64_t n, int64_t k,
                                                         uint8_t* __restrict__ tiled, int64_t units) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int64_t groups = k >> 7;
  const int lane = (int)(u & 63);
  const int64_t tg = u >> 6;
  const int64_t tile = tg / groups;
  const int64_t grp = tg - tile * groups;
  const int64_t row = tile * 16 + (lane & 15);
  const int64_t blk = grp * 4 + (lane >> 4);
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  if (row < n) v = *reinterpret_cast<const u32x4*>(codes + row * (k >> 1) + blk * 16);
  *reinterpret_cast<u32x4*>(tiled + u * 16) = v;
}

// Row-layout scales [n, k/32] -> tiled scales: unit (16 bytes) u of the output, with
// u = (row tile * windows + window) * 128 + r, holds scale bytes 16 * window .. + 15 of
// row 128 * tile + r (zero past k/32 and past n). One thread per unit; k/32 is a multiple
// of 4, so the row is read in 4-byte words.
__global__ __launch_bounds__(256) void tile_scales_kernel(const uint8_t* __restrict__ scales, int64_t n, int64_t k,
                                                          uint8_t* __restrict__ tiled, int64_t units) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int64_t kb = k >> 5;
  const int64_t windows = (k + 511) >> 9;
  const int r = (int)(u & 127);
  const int64_t tw = u >> 7;
  const int64_t tile = tw / windows;
  const int64_t w = tw - tile * windows;
  const int64_t row = tile * 128 + r;
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  if (row < n) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(scales + row * kb + w * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (w * 16 + 4 * j < kb) v[j] = src[j];
  }
  *reinterpret_cast<u32x4*>(tiled + u * 16) = v;
}

}  // namespace

hipError_t launch_verify_gemm_act(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                                  const uint8_t* act_codes, const uint8_t* act_scales, int32_t fmt,
                                  int64_t m, float* y, bool tiled, hipStream_t stream) {
  if (tiled) {
    if (fmt == MXS_ACT_FP8) return launch<MXS_ACT_FP8, true>(codes, scales, n, k, act_codes, act_scales, m, y, stream);
    return launch<MXS_ACT_FP4, true>(codes, scales, n, k, act_codes, act_scales, m, y, stream);
  }
  if (fmt == MXS_ACT_FP8) return launch<MXS_ACT_FP8, false>(codes, scales, n, k, act_codes, act_scales, m, y, stream);
  return launch<MXS_ACT_FP4, false>(codes, scales, n, k, act_codes, act_scales, m, y, stream);
}

hipError_t launch_tile_scales(const uint8_t* scales, int64_t n, int64_t k, uint8_t* tiled, hipStream_t stream) {
  const int64_t units = (n + 127) / 128 * ((k + 511) >> 9) * 128;
  tile_scales_kernel<<<dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream>>>(scales, n, k, tiled, units);
  return hipGetLastError();
}

hipError_t launch_tile_codes(const uint8_t* codes, int64_t n, int64_t k, uint8_t* tiled, hipStream_t stream) {
  const int64_t units = (n + 15) / 16 * (k >> 7) * 64;
  tile_codes_kernel<<<dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream>>>(codes, n, k, tiled, units);
  return hipGetLastError();
}

}  // namespace mxs
