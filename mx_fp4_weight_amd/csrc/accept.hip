// spec_accept kernels: one speculative verification cycle per sequence (gfx950).
//
// Rule ("Module 11. Speculative Decoding and Quantization", §4 and the B18
// bridge of §5): p_i, q_i are the softmax laws of the target and draft logit
// rows; draft token x_i is accepted iff u_i < min(1, p_i(x_i)/q_i(x_i)) (0 when
// q_i(x_i) = 0); the first rejection n stops the scan; the final token is
// drawn from (p_n - q_n)+ at a rejection, or from the next-position target law
// p_K when all K drafts survive, by inverse CDF on the supplied u_K.
//
// Three kernels on the caller's stream:
//   stats   grid (rows, chunks): for every 4096-logit chunk of every target
//           and draft row, the chunk max (exact, fp32) and sum exp(z - max)
//           in fp64. This is the one full read of the logits.
//   decide  grid (chunks, sequences): every workgroup combines its sequence's
//           chunk statistics into (max, sum) per row, gathers p_i(x_i) and
//           q_i(x_i) in fp64 (one lane per draft position), takes n = first
//           rejection with a ballot, then sums the final weights w (residual
//           or bonus row) over its own chunk. Chunk 0 writes the decisions.
//   sample  one workgroup per sequence: inclusive scan of the chunk totals,
//           first chunk whose running total exceeds u_K·Z, then a block scan
//           inside that chunk and a per-thread scan to the token.
// All probabilities and prefix sums are fp64; the result can differ from an
// exact-arithmetic draw only when u_K·Z lies within ~1e-15·Z of an interval
// end. Rounding guards: if no crossing is found where the level above
// placed it, the last positive-weight token of that range is taken, so a
// zero-weight token is never returned.
#include "common.hpp"
#include "internal.hpp"

// No FMA contraction: p - q with p = e_t/S_t must be exactly 0 when the target
// and draft rows are equal, and the decide and sample kernels must compute
// bit-identical weights.
#pragma clang fp contract(off)

namespace mxs {
namespace {

constexpr int kThreads = 256;
constexpr int kPer = 16;
constexpr int kChunk = kThreads * kPer;  // 4096 logits per chunk
constexpr int kMaxRows = 65;             // 2 * 32 + 1 rows per sequence

struct Decision {
  int32_t n;      // accepted drafts, or -1 for a refused sequence
  int32_t pad;
  double mt, inv_st;  // target row n: max and 1/sum
  double md, inv_sd;  // draft row n (n < kd)
};

struct Workspace {
  float* cmax;     // [rows][chunks]
  double* csum;    // [rows][chunks]
  int32_t* cbad;   // [rows][chunks]
  Decision* dec;   // [b]
  double* zres;    // [b][chunks] chunk totals of the final weights
  double* zp;      // [b][chunks] chunk totals of p_n (zero-residual fallback)
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  size_t cmax, csum, cbad, dec, zres, zp, total;
};

inline Layout layout(int64_t b, int64_t kd, int64_t v) {
  const int64_t rows = b * (2 * kd + 1);
  const int64_t chunks = (v + kChunk - 1) / kChunk;
  Layout L;
  size_t off = 0;
  L.cmax = off;
  off = align256(off + sizeof(float) * rows * chunks);
  L.csum = off;
  off = align256(off + sizeof(double) * rows * chunks);
  L.cbad = off;
  off = align256(off + sizeof(int32_t) * rows * chunks);
  L.dec = off;
  off = align256(off + sizeof(Decision) * b);
  L.zres = off;
  off = align256(off + sizeof(double) * b * chunks);
  L.zp = off;
  off = align256(off + sizeof(double) * b * chunks);
  L.total = off;
  return L;
}

// Logit row j of sequence s: rows 0..kd are target rows, kd+1..2kd draft rows.
__device__ inline const float* row_ptr(const float* target, const float* draft, int64_t s, int kd,
                                       int j, int64_t v) {
  if (j <= kd) return target + ((size_t)s * (kd + 1) + j) * (size_t)v;
  return draft + ((size_t)s * kd + (j - kd - 1)) * (size_t)v;
}

// ---------------------------------------------------------------- stats
template <bool kVec4>
__global__ __launch_bounds__(kThreads) void stats_kernel(const float* __restrict__ target,
                                                         const float* __restrict__ draft, int kd,
                                                         int v, int chunks, Workspace ws) {
  __shared__ double lds_d[kThreads / kWave];
  __shared__ float lds_f[kThreads / kWave];
  __shared__ int lds_i[kThreads / kWave];
  const int64_t rowg = blockIdx.x;  // row index over all sequences
  const int per_seq = 2 * kd + 1;
  const int64_t s = rowg / per_seq;
  const int j = (int)(rowg % per_seq);
  const int c = blockIdx.y;
  const float* z = row_ptr(target, draft, s, kd, j, v);
  const int base = c * kChunk;

  float vals[kPer];
  if constexpr (kVec4) {
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const int e = base + 4 * (threadIdx.x + kThreads * q);
      f32x4 t = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (e < v) t = *reinterpret_cast<const f32x4*>(z + e);  // v % 4 == 0: whole vector in range
      vals[4 * q + 0] = t[0];
      vals[4 * q + 1] = t[1];
      vals[4 * q + 2] = t[2];
      vals[4 * q + 3] = t[3];
    }
  } else {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = base + threadIdx.x + kThreads * q;
      vals[q] = e < v ? z[e] : -INFINITY;
    }
  }
  float mx = -INFINITY;
  int bad = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    bad |= (vals[q] != vals[q]) | (vals[q] == INFINITY);
    mx = fmaxf(mx, vals[q]);
  }
  mx = block_max<kThreads>(mx, lds_f);
  bad = block_or<kThreads>(bad, lds_i);
  double acc = 0.0;
  if (mx != -INFINITY && !bad) {
    const double m64 = (double)mx;
#pragma unroll
    for (int q = 0; q < kPer; ++q) acc += exp_neg_f64((double)vals[q] - m64);
  }
  acc = block_sum_f64<kThreads>(acc, lds_d);
  if (threadIdx.x == 0) {
    const size_t o = (size_t)rowg * chunks + c;
    ws.cmax[o] = mx;
    ws.csum[o] = acc;
    ws.cbad[o] = bad;
  }
}

// p_n(t) and the final weight of token t: residual (p - q)+, or p for the bonus row.
struct FinalRows {
  const float* zt;
  const float* zd;  // nullptr for the bonus row
  double mt, inv_st, md, inv_sd;
};

__device__ inline void weights_at(const FinalRows& fr, int t, double& w_final, double& w_p) {
  const double p = exp_neg_f64((double)fr.zt[t] - fr.mt) * fr.inv_st;
  w_p = p;
  if (fr.zd) {
    const double q = exp_neg_f64((double)fr.zd[t] - fr.md) * fr.inv_sd;
    const double d = p - q;
    w_final = d > 0.0 ? d : 0.0;
  } else {
    w_final = p;
  }
}

// ---------------------------------------------------------------- decide + chunk totals
__global__ __launch_bounds__(kThreads) void decide_kernel(
    const float* __restrict__ target, const float* __restrict__ draft,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms, int kd, int v,
    int chunks, Workspace ws, int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_num,
    int32_t* __restrict__ flags) {
  __shared__ double smax[kMaxRows];
  __shared__ double ssum[kMaxRows];
  __shared__ int sbad[kMaxRows];
  __shared__ double lds_d[kThreads / kWave];
  __shared__ int s_n;
  const int c = blockIdx.x;
  const int64_t s = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int per_seq = 2 * kd + 1;

  // 1. per-row max and sum over the chunk statistics: one wave per row
  for (int j = wave; j < per_seq; j += kThreads / kWave) {
    const size_t o = ((size_t)s * per_seq + j) * chunks;
    float m = -INFINITY;
    int bad = 0;
    for (int cc = lane; cc < chunks; cc += kWave) {
      m = fmaxf(m, ws.cmax[o + cc]);
      bad |= ws.cbad[o + cc];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      m = fmaxf(m, __shfl_xor(m, off));
      bad |= __shfl_xor(bad, off);
    }
    bad |= (m == -INFINITY);
    double sum = 0.0;
    if (!bad) {
      const double m64 = (double)m;
      for (int cc = lane; cc < chunks; cc += kWave) {
        const double cs = ws.csum[o + cc];
        if (cs > 0.0) sum += cs * exp_neg_f64((double)ws.cmax[o + cc] - m64);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane == 0) {
      smax[j] = (double)m;
      ssum[j] = sum;
      sbad[j] = bad;
    }
  }
  __syncthreads();

  // 2. decisions: lane i of wave 0 tests draft position i; n = first rejection
  if (wave == 0) {
    int bad = 0;
    for (int j = lane; j < per_seq; j += kWave) bad |= sbad[j];
    bad = __any(bad);
    int f = 0;
    bool acc = true;
    int32_t x = -1;
    if (!bad && lane < kd) {
      x = tokens[(size_t)s * kd + lane];
      double a = 0.0;
      if (x < 0 || x >= v) {
        f |= MXS_FLAG_TOKEN_RANGE;
      } else {
        const float zt = row_ptr(target, draft, s, kd, lane, v)[x];
        const float zd = row_ptr(target, draft, s, kd, kd + 1 + lane, v)[x];
        const double q = exp_neg_f64((double)zd - smax[kd + 1 + lane]) / ssum[kd + 1 + lane];
        const double p = exp_neg_f64((double)zt - smax[lane]) / ssum[lane];
        if (q == 0.0) {
          f |= MXS_FLAG_Q_ZERO;
        } else {
          a = p / q;
          a = a < 1.0 ? a : 1.0;
        }
      }
      acc = (double)uniforms[(size_t)s * (kd + 1) + lane] < a;
    }
    const unsigned long long rej = __ballot(!acc);  // lanes >= kd vote "accept"
    const int n = bad ? -1 : (rej ? __ffsll(rej) - 1 : kd);
    if (lane > n) f = 0;  // positions after the first rejection are not examined
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) f |= __shfl_xor(f, off);
    if (lane == 0) s_n = n;
    if (c == 0) {
      // accepted drafts, then -1; slot n (the final draw) is written by the sample kernel
      int32_t* out = out_tokens + (size_t)s * (kd + 1);
      if (lane <= kd) {
        if (n < 0 || lane > n) out[lane] = -1;
        else if (lane < n) out[lane] = x;
      }
      if (lane == 0) {
        out_num[s] = n < 0 ? 0 : n;
        Decision d;
        d.n = n;
        d.pad = 0;
        const int nn = n < 0 ? 0 : n;
        d.mt = smax[nn];
        d.inv_st = 1.0 / ssum[nn];
        d.md = (n >= 0 && n < kd) ? smax[kd + 1 + n] : 0.0;
        d.inv_sd = (n >= 0 && n < kd) ? 1.0 / ssum[kd + 1 + n] : 0.0;
        ws.dec[s] = d;
        if (bad) raise_flag(flags, MXS_FLAG_NONFINITE);
        else if (f) raise_flag(flags, f);
      }
    }
  }
  __syncthreads();

  // 3. chunk total of the final weights: thread totals in token order, then
  // the same block scan the sample kernel uses, so both see identical totals
  const int n = s_n;
  double a = 0.0, b = 0.0;
  if (n >= 0) {
    FinalRows fr;
    fr.zt = row_ptr(target, draft, s, kd, n, v);
    fr.zd = n < kd ? row_ptr(target, draft, s, kd, kd + 1 + n, v) : nullptr;
    fr.mt = smax[n];
    fr.inv_st = 1.0 / ssum[n];
    fr.md = n < kd ? smax[kd + 1 + n] : 0.0;
    fr.inv_sd = n < kd ? 1.0 / ssum[kd + 1 + n] : 0.0;
    const int t0 = c * kChunk + threadIdx.x * kPer;
    for (int j = 0; j < kPer; ++j) {
      const int t = t0 + j;
      if (t < v) {
        double wf, wp;
        weights_at(fr, t, wf, wp);
        a += wf;
        b += wp;
      }
    }
  }
  a = block_inclusive_scan_f64<kThreads>(a, lds_d);
  b = block_inclusive_scan_f64<kThreads>(b, lds_d);
  if (threadIdx.x == kThreads - 1) {
    ws.zres[s * chunks + c] = a;
    ws.zp[s * chunks + c] = b;
  }
}

// ---------------------------------------------------------------- sample
constexpr int kNone = 0x7fffffff;

__global__ __launch_bounds__(kThreads) void sample_kernel(
    const float* __restrict__ target, const float* __restrict__ draft,
    const float* __restrict__ uniforms, int kd, int v, int chunks, Workspace ws,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ flags) {
  __shared__ double lds_scan[kThreads / kWave];
  __shared__ double s_incl[kThreads];
  __shared__ int s_first, s_last;
  const int64_t s = blockIdx.x;
  const Decision d = ws.dec[s];
  const int n = d.n;
  if (n < 0) return;
  FinalRows fr;
  fr.zt = row_ptr(target, draft, s, kd, n, v);
  fr.zd = n < kd ? row_ptr(target, draft, s, kd, kd + 1 + n, v) : nullptr;
  fr.mt = d.mt;
  fr.inv_st = d.inv_st;
  fr.md = d.md;
  fr.inv_sd = d.inv_sd;
  const int tid = threadIdx.x;

  // ---- level 1: chunks. Z = running total over rounds of 256 chunk totals.
  const double* zr = ws.zres + s * chunks;
  bool use_p = false;
  double Z = 0.0;
  for (int pass = 0; pass < 2; ++pass) {
    double carry = 0.0;
    for (int c0 = 0; c0 < chunks; c0 += kThreads) {
      const int cc = c0 + tid;
      const double incl = carry + block_inclusive_scan_f64<kThreads>(cc < chunks ? zr[cc] : 0.0, lds_scan);
      if (tid == kThreads - 1) s_incl[0] = incl;
      __syncthreads();
      carry = s_incl[0];
      __syncthreads();
    }
    Z = carry;
    if (Z > 0.0 || pass == 1) break;
    // zero residual mass (rounding): draw from p_n instead
    use_p = true;
    zr = ws.zp + s * chunks;
    if (n < kd && tid == 0) raise_flag(flags, MXS_FLAG_RESIDUAL_ZERO);
  }
  const double uz = (double)uniforms[(size_t)s * (kd + 1) + kd] * Z;

  // first positive chunk whose running total exceeds u·Z, and the total before it
  if (tid == 0) {
    s_first = kNone;
    s_last = -1;
  }
  __syncthreads();
  double carry = 0.0, base = 0.0;
  int c = kNone;
  for (int c0 = 0; c0 < chunks; c0 += kThreads) {
    const int cc = c0 + tid;
    const double zc = cc < chunks ? zr[cc] : 0.0;
    const double incl = carry + block_inclusive_scan_f64<kThreads>(zc, lds_scan);
    s_incl[tid] = incl;
    if (cc < chunks && zc > 0.0) {
      if (uz < incl) atomicMin(&s_first, cc);
      atomicMax(&s_last, cc);
    }
    __syncthreads();
    c = s_first;
    if (c != kNone) {
      base = c > c0 ? s_incl[c - c0 - 1] : carry;
      break;
    }
    carry = s_incl[kThreads - 1];
    __syncthreads();
  }
  const bool found = c != kNone;
  if (!found) c = s_last;  // no crossing (u >= 1 or rounding): last chunk with positive weight
  if (c < 0) return;       // a valid row always has positive mass
  __syncthreads();

  // ---- level 2: threads of chunk c (same thread totals and scan as the decide kernel)
  const int t0 = c * kChunk + tid * kPer;
  double wl[kPer];
  double tau = 0.0;
  int lastpos = -1;
  for (int j = 0; j < kPer; ++j) {
    const int t = t0 + j;
    double wf = 0.0, wp = 0.0;
    if (t < v) weights_at(fr, t, wf, wp);
    wl[j] = use_p ? wp : wf;
    tau += wl[j];
    if (wl[j] > 0.0) lastpos = t;
  }
  const double sincl = block_inclusive_scan_f64<kThreads>(tau, lds_scan);
  s_incl[tid] = sincl;
  if (tid == 0) {
    s_first = kNone;
    s_last = -1;
  }
  __syncthreads();
  if (found && tau > 0.0 && uz < base + sincl) atomicMin(&s_first, tid);
  if (lastpos >= 0) atomicMax(&s_last, lastpos);
  __syncthreads();
  int32_t* out = out_tokens + (size_t)s * (kd + 1) + n;
  const int ti = s_first;
  if (ti == kNone) {  // fallback chunk, or rounding: last positive token of the chunk
    if (tid == 0) *out = s_last;
    return;
  }
  if (tid != ti) return;
  // ---- level 3: tokens of thread ti
  const double before = base + (ti > 0 ? s_incl[ti - 1] : 0.0);
  double run = 0.0;
  int pick = -1;
  for (int j = 0; j < kPer; ++j) {
    run += wl[j];
    if (pick < 0 && wl[j] > 0.0 && uz < before + run) pick = t0 + j;
  }
  *out = pick >= 0 ? pick : lastpos;
}

}  // namespace

size_t accept_workspace_bytes(int64_t b, int64_t kd, int64_t v) { return layout(b, kd, v).total; }

hipError_t launch_spec_accept(const float* target, const float* draft, const int32_t* tokens,
                              const float* uniforms, int32_t b, int32_t kd, int32_t v,
                              int32_t* out_tokens, int32_t* out_num, void* workspace,
                              int32_t* flags, bool vec4, hipStream_t stream) {
  const int chunks = (v + kChunk - 1) / kChunk;
  const Layout L = layout(b, kd, v);
  char* base = static_cast<char*>(workspace);
  Workspace ws;
  ws.cmax = reinterpret_cast<float*>(base + L.cmax);
  ws.csum = reinterpret_cast<double*>(base + L.csum);
  ws.cbad = reinterpret_cast<int32_t*>(base + L.cbad);
  ws.dec = reinterpret_cast<Decision*>(base + L.dec);
  ws.zres = reinterpret_cast<double*>(base + L.zres);
  ws.zp = reinterpret_cast<double*>(base + L.zp);
  const int64_t rows = (int64_t)b * (2 * kd + 1);
  dim3 g1((unsigned)rows, (unsigned)chunks);
  if (vec4)
    stats_kernel<true><<<g1, dim3(kThreads), 0, stream>>>(target, draft, kd, v, chunks, ws);
  else
    stats_kernel<false><<<g1, dim3(kThreads), 0, stream>>>(target, draft, kd, v, chunks, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decide_kernel<<<dim3((unsigned)chunks, (unsigned)b), dim3(kThreads), 0, stream>>>(
      target, draft, tokens, uniforms, kd, v, chunks, ws, out_tokens, out_num, flags);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  sample_kernel<<<dim3((unsigned)b), dim3(kThreads), 0, stream>>>(target, draft, uniforms, kd, v,
                                                                  chunks, ws, out_tokens, flags);
  return hipGetLastError();
}

}  // namespace mxs
