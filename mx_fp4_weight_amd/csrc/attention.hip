// mxfp4_kv_attention: the verification pass's attention over an MX-FP4 KV cache (gfx950).
//
// Every query position of the pass sees the committed prefix and the new positions its mask
// allows (its own path: a lower-triangular mask for a chain of drafts, ancestor sets for a
// tree; "Module 11. Speculative Decoding and Quantization", §4: the target pass stays causal),
// over keys and values held as MX-FP4 (news page "Next-Gen Speculative Decoding and FP4
// Quantization Shake Up LLM Inference Economics", "Microscaling FP4 (MX-FP4) Integration"):
//   out[t, h] = sum_l softmax_l(scale * q[t, h] . K^[l, h / G]) V^[l, h / G].
//
// The cache is read once per KV head: a workgroup owns one KV head and a range of cache
// entries, and its G * T query rows (the heads sharing that KV head, at every position) all use
// each decoded entry. Each wave walks steps of 32 entries (two halves of 16):
//   * the step's key and value blocks and scales arrive in the wave's LDS ring by direct
//     global-to-LDS loads, two steps ahead of the arithmetic (lane (r, g) brings block g, 32
//     values of d, of entry r of a half: the A-operand order of the MX-FP4 verify GEMM);
//   * E2M1 x 2^(s-127) is decoded to exact bf16 in registers;
//   * S^T = K^ . Q^T with v_mfma_f32_16x16x32_bf16 (queries are the B operand, loaded once);
//   * an online softmax per query row in fp32 (base 2), whose reference maximum moves only when
//     a step exceeds it by more than 2^8, so the output is rescaled rarely;
//   * O^T += V^T . P^T with v_mfma_f32_16x16x32_bf16: the probabilities of the two halves come
//     out of the first product in the B-operand layout of the second (k slots ordered to match);
//     the value rows go to LDS and come back transposed (ds_read_b64_tr_b16) as the A operand;
//     P is split into a bf16 high part and a bf16 remainder (two products), so its rounding
//     stays below 2^-16.
// The four waves of a workgroup are merged in LDS in one round and the workgroup writes a
// partial (max, sum, unnormalised output) per query row; a combine kernel merges the partials of
// all workgroups. Workgroups are numbered so that the KV heads sharing a 128-byte line of the
// cache run on one XCD at the same time (the line is fetched from HBM once).
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace mxs {
namespace {

constexpr int kD = 128;            // head dimension
constexpr int kAttnThreads = 256;  // 4 waves
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kDT = kD / 16;       // 16-wide d tiles of the output
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kStepEntries = 32;   // cache entries a wave takes per step
constexpr int kVRow = kD + 16;     // bf16 per LDS row of a value tile (288 bytes)
constexpr float kMaxLag = 8.f;     // log2 of the largest unnormalised probability
// LDS ring slot of one step: key codes (2 KiB), value codes (2 KiB), key and value scales
// (256 bytes each, the first 128 used)
constexpr int kSlotBytes = 4096 + 512;
constexpr int kDmaPerStep = 6;     // direct-to-LDS loads per step and wave
constexpr int kLgkmZero = 0xC07F;  // s_waitcnt lgkmcnt(0), vmcnt and expcnt left alone

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct AttnArgs {
  const uint16_t* q;                // [b, T, Hq, d]
  const uint8_t *kc, *ks, *vc, *vs; // [b, cap, Hkv, d/2], [b, cap, Hkv, d/32]
  const int32_t* ctx;               // [b]
  float* part;                      // [b, Hkv, splits, rows_pad, 2 + d]
  int t, hq, hkv, g, rows;          // rows = T * G query rows per KV head
  int64_t cap, max_len;
  int chunk, splits;
  int rows_pad;                     // rows per partial block (16 for up to 16 rows, else 32 per group)
  float scale_log2;                 // scale * log2 e
  uint64_t mask[kMaxAttnPositions]; // bit r of mask[t]: position t sees new position r
};

__device__ inline float e8m0_f32(uint32_t s) {
  uint32_t bits = s << 23;
  bits = (s == 0u) ? 0x00400000u : bits;
  bits = (s == 255u) ? 0x7fc00000u : bits;
  return __uint_as_float(bits);
}

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4 of the 8-byte
// pieces addressed by lanes 4 j + i / 4, j = 0..3 (a 4 x 16 block read back as 16 x 4).
__device__ inline s16x4 tr_read(const __bf16* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<__bf16*>(p)));
  return __builtin_bit_cast(s16x4, v);
}

__device__ inline bf16x8 dec8(uint32_t c, float sc) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 3);
  bf16x8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

// QT query tiles of 16 rows (rows = T * G <= 16 * QT).
template <int QT>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_kernel(const AttnArgs a) {
  // per wave: the step's value tile as rows [entry][d] (kVRow bf16 per row: the padding keeps the
  // transposed reads of four rows on distinct banks); after the loop it holds two waves' scaled
  // outputs for the merge
  constexpr int kWaveVt = kStepEntries * kVRow;
  constexpr int kVtBytes = kAttnWaves * kWaveVt * 2;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kVtBytes];
  // the two slots of every wave's ring are separate arrays, so the compiler can tell that a
  // load into one slot does not write what is being read from the other
  __shared__ __attribute__((aligned(16))) unsigned char ring0[kAttnWaves * kSlotBytes];
  __shared__ __attribute__((aligned(16))) unsigned char ring1[kAttnWaves * kSlotBytes];
  __shared__ float mred[kAttnWaves][QT * 16], sred[kAttnWaves][QT * 16];
  __bf16* vt = reinterpret_cast<__bf16*>(lds);
  // Work item of this workgroup, KV head fastest. Workgroups i and i + 8 run on the same XCD, so
  // each XCD takes a contiguous range of work items: the two heads whose 64-byte blocks share a
  // 128-byte line of the cache run on one XCD at about the same time, and its L2 fetches the
  // line once.
  const int nwg = gridDim.x * gridDim.y * gridDim.z;
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int nwg8 = nwg & ~7;
  const int item = lin < nwg8 ? (lin & 7) * (nwg8 >> 3) + (lin >> 3) : lin;
  const int h = item % a.hkv;         // KV head
  const int rest = item / a.hkv;
  const int groups = gridDim.y / a.hkv;
  const int rg = rest % groups;       // group of 16 QT query rows (rows past 32 take more groups)
  const int split = (rest / groups) % a.splits;
  const int64_t s = rest / groups / a.splits;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r = lane & 15;   // A: entry of a half step / B, C: query row of the tile
  const int g = lane >> 4;   // which 32-value block of d / which entries of the C tile
  const int ctx = __builtin_amdgcn_readfirstlane(a.ctx[s]);  // one value per workgroup
  const bool seq_ok = ctx >= 0 && (int64_t)ctx + a.t <= a.max_len;
  const int len = seq_ok ? ctx + a.t : 0;
  const int p0 = split * a.chunk;
  const int p1 = min(p0 + a.chunk, len);

  // queries: B operand of slice dd for row 16 qt + r = d values 32 g + 8 dd .. + 7 (zero past rows)
  bf16x8 qb[QT][4];
  uint64_t qmask[QT];  // new positions this lane's row (C column) sees; 0 for padding rows
  bool qrow[QT];       // the row is a real query row
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = 16 * QT * rg + 16 * qt + r;
    const int t = row / a.g, gi = row - t * a.g;
    const bool ok = row < a.rows;
    qrow[qt] = ok;
    qmask[qt] = ok ? a.mask[t] : 0ull;
    // padding rows load row 0 and keep zeros (no load sits on one side of a branch)
    const uint16_t* qp = a.q + (((size_t)s * a.t + (ok ? t : 0)) * a.hq + (size_t)h * a.g + (ok ? gi : 0)) * kD + 32 * g;
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qp + 8 * dd);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = ok ? v[i] : 0u;
      qb[qt][dd] = __builtin_bit_cast(bf16x8, v);
    }
  }

  float m_run[QT], s_run[QT];
  f32x4 oacc[QT][kDT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = -INFINITY;
    s_run[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) oacc[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const size_t ent = (size_t)a.hkv * (kD / 2);   // code bytes per cache entry
  const size_t sent = (size_t)a.hkv * (kD / 32); // scale bytes per cache entry
  const uint8_t* kc = a.kc + (size_t)s * a.cap * ent + (size_t)h * (kD / 2);
  const uint8_t* vc = a.vc + (size_t)s * a.cap * ent + (size_t)h * (kD / 2);
  const uint8_t* ks = a.ks + (size_t)s * a.cap * sent + (size_t)h * (kD / 32);
  const uint8_t* vs = a.vs + (size_t)s * a.cap * sent + (size_t)h * (kD / 32);
  __bf16* my_vt = vt + wave * kWaveVt;
  bf16x8* const vt8 = reinterpret_cast<bf16x8*>(lds);
  const int vt8_row = (wave * kWaveVt + r * kVRow + 32 * g) / 8;  // this lane's row r, block g
  // this lane's transposed-read address of value rows 4 g + r / 4 (and 16 + that) at column
  // 4 (r % 4) of each 16-wide d tile: lane (r, g) receives V[4 g + j][16 dt + r], j = 0..3, the
  // A operand of O^T = V^T P^T for entries 4 g .. 4 g + 3
  const __bf16* my_vtr = my_vt + (4 * g + (r >> 2)) * kVRow + 4 * (r & 3);

  // The cache entries stream into a two-slot LDS ring per wave by direct global-to-LDS loads
  // (kDmaPerStep per step). Each step's descriptors end at the chunk's last entry, so entries
  // past it read as zeros (codes and scales 0: decoded values 0) and move no data.
  unsigned char* const my_slot0 = ring0 + wave * kSlotBytes;
  unsigned char* const my_slot1 = ring1 + wave * kSlotBytes;
  auto dma = [&](int t, unsigned char* dst) {
    // entries of the step inside the chunk (one value per wave: the descriptors live in scalars)
    const int nv = __builtin_amdgcn_readfirstlane(max(0, min(kStepEntries, p1 - t)));
    const int tc = nv > 0 ? t : 0;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kc + (size_t)tc * ent, (uint32_t)nv * (uint32_t)ent);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vc + (size_t)tc * ent, (uint32_t)nv * (uint32_t)ent);
    const __amdgpu_buffer_rsrc_t ksr = make_rsrc(ks + (size_t)tc * sent, (uint32_t)nv * (uint32_t)sent);
    const __amdgpu_buffer_rsrc_t vsr = make_rsrc(vs + (size_t)tc * sent, (uint32_t)nv * (uint32_t)sent);
    // codes: lane (r, g) of half hf brings block g of entry 16 hf + r to its own 16 bytes
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint32_t off = opaque((uint32_t)(16 * hf + r) * (uint32_t)ent + 16u * (uint32_t)g);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (__attribute__((address_space(3))) void*)(dst + hf * 1024), 16,
                                               off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (__attribute__((address_space(3))) void*)(dst + 2048 + hf * 1024),
                                               16, off, 0, 0, 0);
    }
    // scales: lane l < 32 brings the 4 block scales of entry l (lanes past 32 read nothing)
    const uint32_t so = opaque(lane < kStepEntries ? (uint32_t)lane * (uint32_t)sent : kOutOfRange);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ksr, (__attribute__((address_space(3))) void*)(dst + 4096), 4, so, 0, 0,
                                             0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vsr, (__attribute__((address_space(3))) void*)(dst + 4096 + 256), 4, so,
                                             0, 0, 0);
  };
  struct Half {
    u32x4 kw, vw;
    uint32_t ksb, vsb;
  };
  auto read_slot = [&](const unsigned char* src, Half (&o)[2]) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      o[hf].kw = *reinterpret_cast<const u32x4*>(src + hf * 1024 + lane * 16);
      o[hf].vw = *reinterpret_cast<const u32x4*>(src + 2048 + hf * 1024 + lane * 16);
      o[hf].ksb = src[4096 + (16 * hf + r) * 4 + g];
      o[hf].vsb = src[4096 + 256 + (16 * hf + r) * 4 + g];
    }
  };
  // One step of 32 entries from cur. kFull: every entry lies in the committed prefix, so every
  // entry is live and visible to every query row (padding rows included: their outputs are
  // never written and their scores are finite), and the masks and guards drop out.
  auto step = [&](int tb, Half (&cur)[2], auto full_c) {
    constexpr bool kFull = decltype(full_c)::value;
    // value rows 16 hf + r, d 32 g .. 32 g + 31, decoded to exact bf16 (indexed from the array
    // itself: a long chain of pointer steps loses the compiler's knowledge of which LDS array is
    // written, and every such store would then wait for the ring's loads)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const float vsf = e8m0_f32(cur[hf].vsb);
#pragma unroll
      for (int dd = 0; dd < 4; ++dd)
        vt8[vt8_row + hf * (16 * kVRow / 8) + dd] = dec8(cur[hf].vw[dd], vsf);
    }
    // scores S^T[entry 16 hf + 4 g + i][row c] for each query tile (unscaled)
    f32x4 sc[QT][2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const float ksf = e8m0_f32(cur[hf].ksb);
      bf16x8 ka[4];
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) ka[dd] = dec8(cur[hf].kw[dd], ksf);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[dd], qb[qt][dd], acc, 0, 0, 0);
        sc[qt][hf] = acc;
      }
    }
    // visibility (partial steps) and each row's step maximum in base-2 units
    bool vis[QT][2][4];
    float mt[QT];
    bool grow = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mr = -INFINITY;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (kFull) {
            vis[qt][hf][i] = true;
          } else {
            const int ei = tb + 16 * hf + 4 * g + i;
            // ei - ctx < T <= 64 for every entry below len; the test is branch free
            const bool seen = (qmask[qt] >> ((uint32_t)(ei - ctx) & 63u)) & 1ull;
            vis[qt][hf][i] = qrow[qt] & (ei < len) & ((ei < ctx) | seen);
          }
          mr = fmaxf(mr, vis[qt][hf][i] ? sc[qt][hf][i] : -INFINITY);
        }
      mr = fmaxf(mr, __shfl_xor(mr, 16));
      mr = fmaxf(mr, __shfl_xor(mr, 32));
      mt[qt] = mr * a.scale_log2;
      grow |= mt[qt] > m_run[qt] + kMaxLag;
    }
    // The reference maximum of a row moves only when the step's maximum exceeds it by more than
    // kMaxLag (in log2 units), so probabilities stay below 2^kMaxLag and the output is rescaled
    // rarely; the softmax is the same for any reference, only its rounding differs.
    if (__any(grow)) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float mn = fmaxf(m_run[qt], mt[qt]);
        const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[qt] - mn);
        m_run[qt] = mn;
        s_run[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) oacc[qt][dt] *= alpha;
      }
    }
    // P^T as two bf16 B operands: the high half of each fp32 probability (truncated) and the
    // remainder rounded to bf16, so the pair is within 2^-16 p of p. k slot 8 g + j holds entry
    // 4 g + j (j < 4) or 16 + 4 g + j - 4 (j >= 4).
    u32x4 ph[QT], pl[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        float pp[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int hf = (j + k) >> 2, i = (j + k) & 3;
          float p = __builtin_amdgcn_exp2f(fmaf(sc[qt][hf][i], a.scale_log2, -m_run[qt]));
          if constexpr (!kFull) p = vis[qt][hf][i] ? p : 0.f;
          ps += p;
          pp[k] = p;
        }
        const uint32_t b0 = __float_as_uint(pp[0]) & 0xffff0000u, b1 = __float_as_uint(pp[1]) & 0xffff0000u;
        ph[qt][j >> 1] = (b0 >> 16) | b1;
        const f32x2 lo = {pp[0] - __uint_as_float(b0), pp[1] - __uint_as_float(b1)};
        pl[qt][j >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
      }
      s_run[qt] += ps;
    }
    // O^T += V^T P^T, 16 d values per product, the value tile read back transposed
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
      const s16x4 v0 = tr_read(my_vtr + 16 * dt);
      const s16x4 v1 = tr_read(my_vtr + 16 * kVRow + 16 * dt);
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        oacc[qt][dt] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, __builtin_bit_cast(bf16x8, ph[qt]), oacc[qt][dt], 0, 0, 0);
        oacc[qt][dt] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, __builtin_bit_cast(bf16x8, pl[qt]), oacc[qt][dt], 0, 0, 0);
      }
    }
  };

  // Step j: wait for its loads (step j + 1 stays in flight), copy it from its slot to
  // registers, refill the slot with step j + 2, compute. Two steps are in flight during each
  // step's arithmetic. Every load is issued unconditionally (those of steps past the chunk move
  // nothing), so the count of loads in flight is the same on every path.
  constexpr int kStride = kStepEntries * kAttnWaves;
  const int tb0 = p0 + kStepEntries * wave;
  dma(tb0, my_slot0);
  dma(tb0 + kStride, my_slot1);
  __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * kDmaPerStep));  // the queries (loaded first)
  auto substep = [&](int t, unsigned char* slot) {
    __builtin_amdgcn_s_waitcnt(vmcnt_only(kDmaPerStep));
    Half cur[2];
    read_slot(slot, cur);
    __builtin_amdgcn_s_waitcnt(kLgkmZero);  // the slot's contents are in registers
    dma(t + 2 * kStride, slot);
    if (t < p1) {
      if (t + kStepEntries <= ctx) step(t, cur, std::true_type{});
      else step(t, cur, std::false_type{});
    }
  };
  for (int tb = tb0; tb < p1; tb += 2 * kStride) {
    substep(tb, my_slot0);
    substep(tb + kStride, my_slot1);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));  // no load into the ring outlives the loop

  // Merge the four waves in one round: each scales its output to the workgroup's row maximum
  // and stores it in LDS (the value tiles and the ring are free now: waves 0 and 1 use the
  // value-tile array, waves 2 and 3 a ring slot each); then wave w adds the four waves' values
  // of the output tiles (qt, dt) with (qt * kDT + dt) % 4 == w and writes them.
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float sr = s_run[qt];
    sr += __shfl_xor(sr, 16);
    sr += __shfl_xor(sr, 32);
    if (g == 0) {
      mred[wave][16 * qt + r] = m_run[qt];
      sred[wave][16 * qt + r] = sr;
    }
  }
  __syncthreads();
  float mx[QT], sum[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = 16 * qt + r;
    mx[qt] = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) mx[qt] = fmaxf(mx[qt], mred[w][row]);
    sum[qt] = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w)
      sum[qt] += mx[qt] == -INFINITY ? 0.f : sred[w][row] * __builtin_amdgcn_exp2f(mred[w][row] - mx[qt]);
    const float f = mx[qt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[qt] - mx[qt]);
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) oacc[qt][dt] *= f;
  }
  constexpr int kTiles = QT * kDT;
  static_assert(kVtBytes >= 2 * kTiles * kWave * 16 && kSlotBytes * kAttnWaves >= kTiles * kWave * 16,
                "each wave's scaled output fits its merge region");
  auto obuf = [&](int w) {  // wave w's merge region
    return w == 0 ? reinterpret_cast<f32x4*>(lds)
                  : w == 1 ? reinterpret_cast<f32x4*>(lds) + kTiles * kWave
                           : w == 2 ? reinterpret_cast<f32x4*>(ring0) : reinterpret_cast<f32x4*>(ring1);
  };
  f32x4* const mine = obuf(wave);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) mine[(qt * kDT + dt) * kWave + lane] = oacc[qt][dt];
  __syncthreads();
  float* part = a.part + (((size_t)s * a.hkv + h) * a.splits + split) * (size_t)a.rows_pad * (2 + kD) +
                (size_t)(16 * QT * rg) * (2 + kD);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    // lane (r, g) holds O[row 16 qt + r][d 16 dt + 4 g + i]; padding rows are not written
    if (!qrow[qt]) continue;
    float* pr = part + (size_t)(16 * qt + r) * (2 + kD);
    if (wave == 0 && g == 0) {
      pr[0] = mx[qt];
      pr[1] = sum[qt];
    }
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
      if ((qt * kDT + dt) % kAttnWaves != wave) continue;
      f32x4 o = oacc[qt][dt];
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w)
        if (w != wave) o += obuf(w)[(qt * kDT + dt) * kWave + lane];
      *reinterpret_cast<f32x4*>(pr + 2 + 16 * dt + 4 * g) = o;
    }
  }
}

// One workgroup per query row and KV head, one thread per d element: the workgroups' partials
// merged and normalised. The first kBatch splits' outputs are loaded together with the splits'
// (max, sum) pairs, so up to kBatch splits take one round trip to memory; later splits follow in
// batches of kBatch.
constexpr int kMaxSplits = 512;
constexpr int kBatch = 32;
__global__ __launch_bounds__(kD) void attn_combine_kernel(const AttnArgs a, int rows_pad, float* __restrict__ out,
                                                          int32_t* __restrict__ flags) {
  __shared__ float wsp[kMaxSplits], ssp[kMaxSplits];
  __shared__ float red[kD / kWave];
  const int row = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t s = blockIdx.z;
  const int t = row / a.g, gi = row - t * a.g;
  float* o = out + (((size_t)s * a.t + t) * a.hq + (size_t)h * a.g + gi) * kD;
  const int ctx = a.ctx[s];
  if (!(ctx >= 0 && (int64_t)ctx + a.t <= a.max_len)) {  // refused sequence
    o[threadIdx.x] = __uint_as_float(0x7fc00000u);
    if (threadIdx.x == 0 && row == 0 && h == 0) raise_flag(flags, MXS_FLAG_TOKEN_RANGE);
    return;
  }
  const size_t stride = (size_t)rows_pad * (2 + kD);
  const float* base = a.part + ((size_t)s * a.hkv + h) * a.splits * stride + (size_t)row * (2 + kD);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int splits = a.splits;
  float ov[kBatch];
#pragma unroll
  for (int i = 0; i < kBatch; ++i) ov[i] = base[(size_t)min(i, splits - 1) * stride + 2 + threadIdx.x];
  float mx = -INFINITY;
  for (int sp = threadIdx.x; sp < splits; sp += kD) {
    const f32x2 ms = *reinterpret_cast<const f32x2*>(base + (size_t)sp * stride);
    wsp[sp] = ms[0];
    ssp[sp] = ms[1];
    mx = fmaxf(mx, ms[0]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = fmaxf(red[0], red[1]);
  float sum = 0.f;
  for (int sp = threadIdx.x; sp < splits; sp += kD) {
    const float m = wsp[sp];
    const float w = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mx);
    wsp[sp] = w;
    sum += w * ssp[sp];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  __syncthreads();
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  sum = red[0] + red[1];
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kBatch; ++i)
    if (i < splits) acc += wsp[i] * ov[i];
  for (int b0 = kBatch; b0 < splits; b0 += kBatch) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) ov[i] = base[(size_t)min(b0 + i, splits - 1) * stride + 2 + threadIdx.x];
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (b0 + i < splits) acc += wsp[b0 + i] * ov[i];
  }
  o[threadIdx.x] = acc / sum;
}

}  // namespace

// Query tiles of 16 rows a launch uses (1, 2 or 4).
inline int attn_qtiles(int rows) { return rows <= 16 ? 1 : 2; }
// Groups of 16 * qtiles rows a KV head's rows take (one up to 32 rows, two up to 64).
inline int attn_rgroups(int rows) { return rows <= 16 ? 1 : (rows + 31) / 32; }

// Entries per workgroup: about two workgroups per CU over the sequences and KV heads, in
// multiples of one step of the four waves (128 entries).
inline int attn_chunk(int64_t max_len, int64_t b, int hkv) {
  constexpr int64_t kGrain = (int64_t)kStepEntries * kAttnWaves;
  const int64_t want = (int64_t)2 * device_cus();
  int64_t per = (b * hkv) > 0 ? want / (b * hkv) : 1;
  per = per < 1 ? 1 : (per > kMaxSplits ? kMaxSplits : per);
  int64_t chunk = (max_len + per - 1) / per;
  chunk = (chunk + kGrain - 1) / kGrain * kGrain;
  return (int)(chunk < kGrain ? kGrain : chunk);
}

size_t kv_attention_workspace_bytes(int64_t b, int t, int hq, int hkv, int64_t max_len) {
  const int rows = t * (hq / hkv);
  const int rows_pad = 16 * attn_qtiles(rows) * attn_rgroups(rows);
  const int chunk = attn_chunk(max_len, b, hkv);
  const int64_t splits = (max_len + chunk - 1) / chunk;
  return sizeof(float) * (size_t)b * hkv * splits * rows_pad * (2 + kD);
}

hipError_t launch_kv_attention(const uint16_t* q, const uint8_t* kc, const uint8_t* ks, const uint8_t* vc,
                               const uint8_t* vs, const int32_t* ctx, int32_t b, int32_t t, int32_t hq, int32_t hkv,
                               int64_t cap, int64_t max_len, const uint64_t* masks, float scale, float* out,
                               void* workspace, int32_t* flags, hipStream_t stream) {
  AttnArgs a{};
  a.q = q;
  a.kc = kc;
  a.ks = ks;
  a.vc = vc;
  a.vs = vs;
  a.ctx = ctx;
  a.part = static_cast<float*>(workspace);
  a.t = t;
  a.hq = hq;
  a.hkv = hkv;
  a.g = hq / hkv;
  a.rows = t * a.g;
  a.cap = cap;
  a.max_len = max_len;
  a.chunk = attn_chunk(max_len, b, hkv);
  a.splits = (int)((max_len + a.chunk - 1) / a.chunk);
  a.scale_log2 = scale * kLog2e;
  for (int i = 0; i < t; ++i) a.mask[i] = masks[i];
  const int qt = attn_qtiles(a.rows);
  const int groups = attn_rgroups(a.rows);
  a.rows_pad = 16 * qt * groups;
  const dim3 grid((unsigned)a.splits, (unsigned)(hkv * groups), (unsigned)b);
  if (qt == 1) attn_kernel<1><<<grid, dim3(kAttnThreads), 0, stream>>>(a);
  else attn_kernel<2><<<grid, dim3(kAttnThreads), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows_pad = a.rows_pad;
  attn_combine_kernel<<<dim3((unsigned)a.rows, (unsigned)hkv, (unsigned)b), dim3(kD), 0, stream>>>(a, rows_pad, out,
                                                                                               flags);
  return hipGetLastError();
}

}  // namespace mxs
