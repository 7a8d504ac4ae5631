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
// each decoded entry. Per 16-entry tile a wave
//   * loads the 16 entries' key and value blocks (one 16-byte load per lane: lane (r, g) holds
//     block g (32 values of d) of entry r, the A-operand order of the MX-FP4 verify GEMM) and
//     decodes E2M1 x 2^(s-127) to exact bf16 in registers;
//   * forms S^T = K^ . Q^T with v_mfma_f32_16x16x32_bf16 (queries are the B operand, loaded once);
//   * keeps an online softmax per query row in fp32 (base 2, scores pre-scaled by log2 e);
//   * forms O^T += V^T . P^T with v_mfma_f32_16x16x16_bf16: the probabilities come out of the
//     first product in exactly the B-operand layout of the second; the value tile goes through
//     the wave's own LDS region to be read as the transposed A operand; P is split into a bf16
//     high part and a bf16 remainder (two products), so its rounding stays near 2^-17.
// The four waves of a workgroup are merged in LDS and the workgroup writes a partial (max, sum,
// unnormalised output) per query row; a combine kernel merges the partials of all workgroups.
#include "common.hpp"
#include "internal.hpp"

namespace mxs {
namespace {

constexpr int kD = 128;            // head dimension
constexpr int kAttnThreads = 256;  // 4 waves
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kDT = kD / 16;       // 16-wide d tiles of the output
constexpr float kLog2e = 1.4426950408889634f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

struct AttnArgs {
  const uint16_t* q;                // [b, T, Hq, d]
  const uint8_t *kc, *ks, *vc, *vs; // [b, cap, Hkv, d/2], [b, cap, Hkv, d/32]
  const int32_t* ctx;               // [b]
  float* part;                      // [b, Hkv, splits, rows_pad, 2 + d]
  int t, hq, hkv, g, rows;          // rows = T * G query rows per KV head
  int64_t cap, max_len;
  int chunk, splits;
  float scale_log2;                 // scale * log2 e
  uint64_t mask[kMaxAttnPositions]; // bit r of mask[t]: position t sees new position r
};

__device__ inline float e8m0_f32(uint32_t s) {
  uint32_t bits = s << 23;
  bits = (s == 0u) ? 0x00400000u : bits;
  bits = (s == 255u) ? 0x7fc00000u : bits;
  return __uint_as_float(bits);
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
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(const AttnArgs a) {
  __shared__ __bf16 vt[kAttnWaves][kD * 16];             // per wave: value tile as [d][entry]
  __shared__ f32x4 obuf[QT][kDT][kWave];                 // one wave's scaled output at a time
  __shared__ float mred[kAttnWaves][QT * 16], sred[kAttnWaves][QT * 16];
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t s = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15;   // A: entry of the tile / B, C: query row of the tile
  const int g = lane >> 4;   // which 32-value block of d / which 4 entries of the C tile
  const int ctx = a.ctx[s];
  const bool seq_ok = ctx >= 0 && (int64_t)ctx + a.t <= a.max_len;
  const int len = seq_ok ? ctx + a.t : 0;
  const int p0 = split * a.chunk;
  const int p1 = min(p0 + a.chunk, len);

  // queries: B operand of slice dd for row 16 qt + r = d values 32 g + 8 dd .. + 7 (zero past rows)
  bf16x8 qb[QT][4];
  int qpos[QT];  // query position of this lane's row (C column)
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = 16 * qt + r;
    const int t = row / a.g, gi = row - t * a.g;
    qpos[qt] = row < a.rows ? t : -1;
    const bool ok = row < a.rows;
    const uint16_t* qp = a.q + (((size_t)s * a.t + (ok ? t : 0)) * a.hq + (size_t)h * a.g + (ok ? gi : 0)) * kD + 32 * g;
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) v = *reinterpret_cast<const u32x4*>(qp + 8 * dd);
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
  __bf16* my_vt = vt[wave];

  // this lane's key and value blocks of entry e (entries past the visible range load nothing)
  auto load_tile = [&](int tb, u32x4& kw, u32x4& vw, uint32_t& ksb, uint32_t& vsb) {
    const int e = tb + r;
    kw = u32x4{0u, 0u, 0u, 0u};
    vw = u32x4{0u, 0u, 0u, 0u};
    ksb = 127u;
    vsb = 127u;
    if (tb < p1 && e < len) {
      kw = *reinterpret_cast<const u32x4*>(kc + (size_t)e * ent + 16 * g);
      vw = *reinterpret_cast<const u32x4*>(vc + (size_t)e * ent + 16 * g);
      ksb = ks[(size_t)e * sent + g];
      vsb = vs[(size_t)e * sent + g];
    }
  };
  u32x4 kw, vw;
  uint32_t ksb, vsb;
  load_tile(p0 + 16 * wave, kw, vw, ksb, vsb);
  for (int tb = p0 + 16 * wave; tb < p1; tb += 16 * kAttnWaves) {
    // the next tile's blocks are in flight while this one is computed
    u32x4 kwn, vwn;
    uint32_t ksbn, vsbn;
    load_tile(tb + 16 * kAttnWaves, kwn, vwn, ksbn, vsbn);
    // value tile -> LDS as [d][entry] (zeros for dead entries)
    const float vsf = e8m0_f32(vsb);
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
      const bf16x8 v8 = dec8(vw[dd], vsf);
#pragma unroll
      for (int i = 0; i < 8; ++i) my_vt[(32 * g + 8 * dd + i) * 16 + r] = v8[i];
    }
    // scores S^T[entry 4g + i][row c] for each query tile
    const float ksf = e8m0_f32(ksb);
    bf16x8 ka[4];
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) ka[dd] = dec8(kw[dd], ksf);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[dd], qb[qt][dd], sc, 0, 0, 0);
      // visibility of entry tb + 4g + i for this lane's query row
      float x[4];
      float mt = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ei = tb + 4 * g + i;
        bool vis = qpos[qt] >= 0 && ei < len;
        if (vis && ei >= ctx) vis = (a.mask[qpos[qt]] >> (ei - ctx)) & 1ull;
        x[i] = vis ? sc[i] * a.scale_log2 : -INFINITY;
        mt = fmaxf(mt, x[i]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m_run[qt], mt);
      const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[qt] - mn);
      m_run[qt] = mn;
      float p[4], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = x[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x[i] - mn);
        ps += p[i];
      }
      s_run[qt] = s_run[qt] * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) oacc[qt][dt] *= alpha;
      // P^T as two bf16 B operands: the rounded value and its remainder
      bf16x4 ph, pl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ph[i] = (__bf16)p[i];
        pl[i] = (__bf16)(p[i] - (float)ph[i]);
      }
      const s16x4 bh = __builtin_bit_cast(s16x4, ph), bl = __builtin_bit_cast(s16x4, pl);
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        // A = V^T rows 16 dt + r, entries 4g .. 4g + 3
        const s16x4 va = *reinterpret_cast<const s16x4*>(my_vt + (16 * dt + r) * 16 + 4 * g);
        oacc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, bh, oacc[qt][dt], 0, 0, 0);
        oacc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, bl, oacc[qt][dt], 0, 0, 0);
      }
    }
    kw = kwn;
    vw = vwn;
    ksb = ksbn;
    vsb = vsbn;
  }

  // merge the four waves: each scales its output to the workgroup's row maximum, and wave 0
  // adds the others' in rounds through one LDS buffer
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
  for (int w = 1; w < kAttnWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) obuf[qt][dt][lane] = oacc[qt][dt];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) oacc[qt][dt] += obuf[qt][dt][lane];
    }
    __syncthreads();
  }
  if (wave != 0) return;
  const int rows_pad = 16 * QT;
  float* part = a.part + (((size_t)s * a.hkv + h) * a.splits + split) * (size_t)rows_pad * (2 + kD);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    // lane (r, g) holds O[row 16 qt + r][d 16 dt + 4 g + i]
    float* pr = part + (size_t)(16 * qt + r) * (2 + kD);
    if (g == 0) {
      pr[0] = mx[qt];
      pr[1] = sum[qt];
    }
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
      *reinterpret_cast<f32x4*>(pr + 2 + 16 * dt + 4 * g) = oacc[qt][dt];
  }
}

// One workgroup per query row and KV head, one thread per d element: the workgroups' partials
// merged (their maxima and weights first, all loaded at once; then the weighted outputs, several
// splits' loads in flight per thread) and normalised.
constexpr int kMaxSplits = 512;
__global__ __launch_bounds__(kD) void attn_combine_kernel(const AttnArgs a, int rows_pad, float* __restrict__ out,
                                                          int32_t* __restrict__ flags) {
  __shared__ float wsp[kMaxSplits];
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
  float mx = -INFINITY;
  for (int sp = threadIdx.x; sp < a.splits; sp += kD) {
    const float m = base[sp * stride];
    wsp[sp] = m;
    mx = fmaxf(mx, m);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = fmaxf(red[0], red[1]);
  float sum = 0.f;
  for (int sp = threadIdx.x; sp < a.splits; sp += kD) {
    const float m = wsp[sp];
    const float w = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mx);
    wsp[sp] = w;
    sum += w * base[sp * stride + 1];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  __syncthreads();
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  sum = red[0] + red[1];
  float acc = 0.f;
#pragma unroll 8
  for (int sp = 0; sp < a.splits; ++sp) acc += wsp[sp] * base[sp * stride + 2 + threadIdx.x];
  o[threadIdx.x] = acc / sum;
}

}  // namespace

// Query tiles of 16 rows a launch uses (1, 2 or 4).
inline int attn_qtiles(int rows) { return rows <= 16 ? 1 : (rows <= 32 ? 2 : 4); }

// Entries per workgroup: about two workgroups per CU over the sequences and KV heads, in
// multiples of 64 (each wave walks its 16-entry tiles).
inline int attn_chunk(int64_t max_len, int64_t b, int hkv) {
  const int64_t want = (int64_t)2 * device_cus();
  int64_t per = (b * hkv) > 0 ? want / (b * hkv) : 1;
  per = per < 1 ? 1 : (per > kMaxSplits ? kMaxSplits : per);
  int64_t chunk = (max_len + per - 1) / per;
  chunk = (chunk + 63) / 64 * 64;
  return (int)(chunk < 64 ? 64 : chunk);
}

size_t kv_attention_workspace_bytes(int64_t b, int t, int hq, int hkv, int64_t max_len) {
  const int rows = t * (hq / hkv);
  const int rows_pad = 16 * attn_qtiles(rows);
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
  const dim3 grid((unsigned)a.splits, (unsigned)hkv, (unsigned)b);
  if (qt == 1) attn_kernel<1><<<grid, dim3(kAttnThreads), 0, stream>>>(a);
  else if (qt == 2) attn_kernel<2><<<grid, dim3(kAttnThreads), 0, stream>>>(a);
  else attn_kernel<4><<<grid, dim3(kAttnThreads), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows_pad = qt * 16;
  attn_combine_kernel<<<dim3((unsigned)a.rows, (unsigned)hkv, (unsigned)b), dim3(kD), 0, stream>>>(a, rows_pad, out,
                                                                                               flags);
  return hipGetLastError();
}

}  // namespace mxs
