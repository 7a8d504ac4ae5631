// spec_accept kernels: one speculative verification cycle per sequence (gfx950).
//
// Rule ("Module 11. Speculative Decoding and Quantization", §4 and the B18
// bridge of §5): p_i, q_i are the softmax laws of the target and draft logit
// rows; draft token x_i is accepted iff u_i < min(1, p_i(x_i)/q_i(x_i)) (0 when
// q_i(x_i) = 0); the first rejection n stops the scan; the final token is
// drawn from (p_n - q_n)+ at a rejection, or from the next-position target law
// p_K when all K drafts survive, by inverse CDF on the supplied u_K.
//
// Four kernels on the caller's stream:
//   stats    grid (rows, chunks): per 4096-logit chunk of every target/draft
//            row, the chunk max (exact, fp32) and sum exp(z - max) in fp64.
//            One read of all logits: the vocab-wide normalizers.
//   decide   one wave per sequence: combine chunk stats into (max, sum) per
//            row, gather p_i(x_i), q_i(x_i) in fp64, run the left-to-right
//            test, record n and the row statistics of the final draw.
//   wsum     grid (chunks, sequences): per chunk, the final weights w (residual
//            or bonus row) and their prefix structure; writes the chunk total.
//   sample   one workgroup per sequence: locate u_K · Z among the chunk
//            totals, then inside the chunk among the thread totals, then
//            among the elements; writes t*.
//
// Prefix sums are defined hierarchically and used identically by wsum and
// sample: L = sequential prefix over a thread's 16 consecutive tokens,
// T_i = T_(i-1) + (thread i total) sequentially over the 256 threads of a
// chunk, P_(c+1) = P_c + T_255 over chunks, and C_t = P_c + (T_(i-1) + L_j).
// C is non-decreasing and its value at the end of a thread / chunk is exactly
// the total used one level up, so the crossing always exists where the upper
// level says, and a zero-weight token is never chosen.
#include "common.hpp"
#include "internal.hpp"

#pragma clang fp contract(off)

namespace mxs {
namespace {

constexpr int kThreads = 256;
constexpr int kPer = 16;
constexpr int kChunk = kThreads * kPer;  // 4096 logits per chunk

struct Workspace {
  float* cmax;     // [rows][chunks]
  double* csum;    // [rows][chunks]
  int32_t* cbad;   // [rows][chunks]
  int32_t* nacc;   // [b]  n, or -1 for a refused sequence
  double* rstat;   // [b][4]  (max_t, sum_t, max_d, sum_d) of the final draw's rows
  double* zres;    // [b][chunks]  chunk totals of the final weights
  double* zp;      // [b][chunks]  chunk totals of p_n (zero-residual fallback)
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline Workspace carve(void* base, int64_t b, int64_t kd, int64_t v) {
  const int64_t rows = b * (2 * kd + 1);
  const int64_t chunks = (v + kChunk - 1) / kChunk;
  char* p = static_cast<char*>(base);
  Workspace w;
  size_t off = 0;
  w.cmax = reinterpret_cast<float*>(p + off);
  off = align256(off + sizeof(float) * rows * chunks);
  w.csum = reinterpret_cast<double*>(p + off);
  off = align256(off + sizeof(double) * rows * chunks);
  w.cbad = reinterpret_cast<int32_t*>(p + off);
  off = align256(off + sizeof(int32_t) * rows * chunks);
  w.nacc = reinterpret_cast<int32_t*>(p + off);
  off = align256(off + sizeof(int32_t) * b);
  w.rstat = reinterpret_cast<double*>(p + off);
  off = align256(off + sizeof(double) * 4 * b);
  w.zres = reinterpret_cast<double*>(p + off);
  off = align256(off + sizeof(double) * b * chunks);
  w.zp = reinterpret_cast<double*>(p + off);
  return w;
}

__host__ __device__ inline size_t carve_bytes(int64_t b, int64_t kd, int64_t v) {
  const int64_t rows = b * (2 * kd + 1);
  const int64_t chunks = (v + kChunk - 1) / kChunk;
  size_t off = 0;
  off = align256(off + sizeof(float) * rows * chunks);
  off = align256(off + sizeof(double) * rows * chunks);
  off = align256(off + sizeof(int32_t) * rows * chunks);
  off = align256(off + sizeof(int32_t) * b);
  off = align256(off + sizeof(double) * 4 * b);
  off = align256(off + sizeof(double) * b * chunks);
  off = align256(off + sizeof(double) * b * chunks);
  return off;
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
  const int64_t rowg = blockIdx.x;  // global row index over all sequences
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

// ---------------------------------------------------------------- decide
__global__ __launch_bounds__(kWave) void decide_kernel(
    const float* __restrict__ target, const float* __restrict__ draft,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms, int kd, int v,
    int chunks, Workspace ws, int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_num,
    int32_t* __restrict__ flags) {
  __shared__ double smax[65];
  __shared__ double ssum[65];
  __shared__ int sbad;
  const int64_t s = blockIdx.x;
  const int lane = threadIdx.x;
  const int per_seq = 2 * kd + 1;
  if (lane == 0) sbad = 0;
  __syncthreads();
  for (int j = lane; j < per_seq; j += kWave) {
    const size_t o = ((size_t)s * per_seq + j) * chunks;
    float m = -INFINITY;
    int bad = 0;
    for (int c = 0; c < chunks; ++c) {
      m = fmaxf(m, ws.cmax[o + c]);
      bad |= ws.cbad[o + c];
    }
    double sum = 0.0;
    if (m == -INFINITY) bad = 1;
    if (!bad) {
      const double m64 = (double)m;
      for (int c = 0; c < chunks; ++c) {
        const double cs = ws.csum[o + c];
        if (cs > 0.0) sum += cs * exp_neg_f64((double)ws.cmax[o + c] - m64);
      }
    }
    smax[j] = (double)m;
    ssum[j] = sum;
    if (bad) atomicOr(&sbad, 1);
  }
  __syncthreads();
  int32_t* out = out_tokens + (size_t)s * (kd + 1);
  if (sbad) {
    for (int i = lane; i <= kd; i += kWave) out[i] = -1;
    if (lane == 0) {
      out_num[s] = 0;
      ws.nacc[s] = -1;
      raise_flag(flags, MXS_FLAG_NONFINITE);
    }
    return;
  }
  if (lane != 0) return;
  int f = 0;
  int n = kd;
  const float* u = uniforms + (size_t)s * (kd + 1);
  for (int i = 0; i < kd; ++i) {
    const int32_t x = tokens[(size_t)s * kd + i];
    double a = 0.0;
    if (x < 0 || x >= v) {
      f |= MXS_FLAG_TOKEN_RANGE;
    } else {
      const float zt = row_ptr(target, draft, s, kd, i, v)[x];
      const float zd = row_ptr(target, draft, s, kd, kd + 1 + i, v)[x];
      const double q = exp_neg_f64((double)zd - smax[kd + 1 + i]) / ssum[kd + 1 + i];
      const double p = exp_neg_f64((double)zt - smax[i]) / ssum[i];
      if (q == 0.0) {
        f |= MXS_FLAG_Q_ZERO;
      } else {
        a = p / q;
        a = a < 1.0 ? a : 1.0;
      }
    }
    if ((double)u[i] < a) {
      out[i] = x;
    } else {
      n = i;
      break;
    }
  }
  for (int i = n + 1; i <= kd; ++i) out[i] = -1;
  out_num[s] = n;
  ws.nacc[s] = n;
  double* rs = ws.rstat + 4 * s;
  rs[0] = smax[n];
  rs[1] = ssum[n];
  rs[2] = n < kd ? smax[kd + 1 + n] : 0.0;
  rs[3] = n < kd ? ssum[kd + 1 + n] : 0.0;
  if (f) raise_flag(flags, f);
}

// ---------------------------------------------------------------- final weights
struct FinalRows {
  const float* zt;  // target row n
  const float* zd;  // draft row n, or nullptr for the bonus row
  double mt, st, md, sd;
};

__device__ inline FinalRows final_rows(const float* target, const float* draft, int64_t s, int kd,
                                       int v, int n, const double* rs) {
  FinalRows fr;
  fr.zt = row_ptr(target, draft, s, kd, n, v);
  fr.zd = n < kd ? row_ptr(target, draft, s, kd, kd + 1 + n, v) : nullptr;
  fr.mt = rs[0];
  fr.st = rs[1];
  fr.md = rs[2];
  fr.sd = rs[3];
  return fr;
}

// p_n(t) and the final weight of token t (residual (p - q)+, or p for the bonus row).
__device__ inline void weights_at(const FinalRows& fr, int t, double& w_final, double& w_p) {
  const double p = exp_neg_f64((double)fr.zt[t] - fr.mt) / fr.st;
  w_p = p;
  if (fr.zd) {
    const double q = exp_neg_f64((double)fr.zd[t] - fr.md) / fr.sd;
    const double d = p - q;
    w_final = d > 0.0 ? d : 0.0;
  } else {
    w_final = p;
  }
}

// Thread-local sequential sums of the chunk's 16 consecutive tokens of this thread.
__device__ inline void thread_sums(const FinalRows& fr, int v, int c, double& tot_final,
                                   double& tot_p) {
  const int t0 = c * kChunk + threadIdx.x * kPer;
  double a = 0.0, b = 0.0;
  for (int j = 0; j < kPer; ++j) {
    const int t = t0 + j;
    if (t < v) {
      double wf, wp;
      weights_at(fr, t, wf, wp);
      a = a + wf;
      b = b + wp;
    }
  }
  tot_final = a;
  tot_p = b;
}

__global__ __launch_bounds__(kThreads) void wsum_kernel(const float* __restrict__ target,
                                                        const float* __restrict__ draft, int kd,
                                                        int v, int chunks, Workspace ws) {
  __shared__ double tf[kThreads];
  __shared__ double tp[kThreads];
  const int c = blockIdx.x;
  const int64_t s = blockIdx.y;
  const int n = ws.nacc[s];
  if (n < 0) {
    if (threadIdx.x == 0) {
      ws.zres[s * chunks + c] = 0.0;
      ws.zp[s * chunks + c] = 0.0;
    }
    return;
  }
  const FinalRows fr = final_rows(target, draft, s, kd, v, n, ws.rstat + 4 * s);
  double a, b;
  thread_sums(fr, v, c, a, b);
  tf[threadIdx.x] = a;
  tp[threadIdx.x] = b;
  __syncthreads();
  if (threadIdx.x == 0) {
    double sa = 0.0, sb = 0.0;
    for (int i = 0; i < kThreads; ++i) {
      sa = sa + tf[i];
      sb = sb + tp[i];
    }
    ws.zres[s * chunks + c] = sa;
    ws.zp[s * chunks + c] = sb;
  }
}

// ---------------------------------------------------------------- sample
__global__ __launch_bounds__(kThreads) void sample_kernel(
    const float* __restrict__ target, const float* __restrict__ draft,
    const float* __restrict__ uniforms, int kd, int v, int chunks, Workspace ws,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ flags) {
  __shared__ double T[kThreads];
  __shared__ double s_uz, s_P;
  __shared__ int s_chunk, s_use_p, s_found;
  __shared__ int s_last;
  const int64_t s = blockIdx.x;
  const int n = ws.nacc[s];
  if (n < 0) return;
  const FinalRows fr = final_rows(target, draft, s, kd, v, n, ws.rstat + 4 * s);

  if (threadIdx.x == 0) {
    const double* zr = ws.zres + s * chunks;
    double Z = 0.0;
    for (int c = 0; c < chunks; ++c) Z = Z + zr[c];
    int use_p = 0;
    if (!(Z > 0.0)) {  // zero residual mass: draw from p_n instead
      use_p = 1;
      zr = ws.zp + s * chunks;
      Z = 0.0;
      for (int c = 0; c < chunks; ++c) Z = Z + zr[c];
      if (n < kd) raise_flag(flags, MXS_FLAG_RESIDUAL_ZERO);
    }
    const double uz = (double)uniforms[(size_t)s * (kd + 1) + kd] * Z;
    double P = 0.0;
    int cstar = -1;
    for (int c = 0; c < chunks; ++c) {
      const double next = P + zr[c];
      if (uz < next) {
        cstar = c;
        break;
      }
      P = next;
    }
    int last = -1;
    if (cstar < 0) {  // no crossing (rounding): last chunk holding a positive weight
      for (int c = chunks - 1; c >= 0; --c)
        if (zr[c] > 0.0) {
          last = c;
          break;
        }
    }
    s_uz = uz;
    s_P = P;
    s_chunk = cstar >= 0 ? cstar : last;
    s_found = cstar >= 0;
    s_use_p = use_p;
    s_last = -1;
  }
  __syncthreads();
  const int c = s_chunk;
  const bool use_p = s_use_p;
  if (c < 0) return;  // cannot happen for a valid row (p has positive mass)

  // thread totals of chunk c, identical arithmetic to wsum_kernel
  double a, b;
  thread_sums(fr, v, c, a, b);
  const double mine = use_p ? b : a;
  T[threadIdx.x] = mine;
  __syncthreads();
  if (threadIdx.x == 0) {
    double run = 0.0;
    for (int i = 0; i < kThreads; ++i) {
      run = run + T[i];
      T[i] = run;  // T_i: inclusive sequential prefix of thread totals
    }
  }
  __syncthreads();
  const double P = s_P;
  const double uz = s_uz;
  const int t0 = c * kChunk + threadIdx.x * kPer;
  int32_t* out = out_tokens + (size_t)s * (kd + 1) + n;
  if (s_found) {
    const double before = threadIdx.x > 0 ? T[threadIdx.x - 1] : 0.0;
    const bool here = uz < P + T[threadIdx.x];
    const bool prev = threadIdx.x > 0 ? (uz < P + before) : false;
    if (here && !prev) {
      double L = 0.0;
      int pick = -1, lastpos = -1;
      for (int j = 0; j < kPer; ++j) {
        const int t = t0 + j;
        if (t >= v) break;
        double wf, wp;
        weights_at(fr, t, wf, wp);
        const double w = use_p ? wp : wf;
        L = L + w;
        if (w > 0.0) lastpos = t;
        if (uz < P + (before + L)) {
          pick = t;
          break;
        }
      }
      // the crossing exists at this thread's end by construction; keep a guard
      *out = pick >= 0 ? pick : lastpos;
    }
  } else {
    // fallback: the last token of chunk c with positive weight
    int lastpos = -1;
    for (int j = 0; j < kPer; ++j) {
      const int t = t0 + j;
      if (t >= v) break;
      double wf, wp;
      weights_at(fr, t, wf, wp);
      if ((use_p ? wp : wf) > 0.0) lastpos = t;
    }
    if (lastpos >= 0) atomicMax(&s_last, lastpos);
    __syncthreads();
    if (threadIdx.x == 0) *out = s_last;
  }
}

}  // namespace

size_t accept_workspace_bytes(int64_t b, int64_t kd, int64_t v) { return carve_bytes(b, kd, v); }

hipError_t launch_spec_accept(const float* target, const float* draft, const int32_t* tokens,
                              const float* uniforms, int32_t b, int32_t kd, int32_t v,
                              int32_t* out_tokens, int32_t* out_num, void* workspace,
                              int32_t* flags, bool vec4, hipStream_t stream) {
  const int chunks = (v + kChunk - 1) / kChunk;
  const Workspace ws = carve(workspace, b, kd, v);
  const int64_t rows = (int64_t)b * (2 * kd + 1);
  dim3 g1((unsigned)rows, (unsigned)chunks);
  if (vec4)
    stats_kernel<true><<<g1, dim3(kThreads), 0, stream>>>(target, draft, kd, v, chunks, ws);
  else
    stats_kernel<false><<<g1, dim3(kThreads), 0, stream>>>(target, draft, kd, v, chunks, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decide_kernel<<<dim3((unsigned)b), dim3(kWave), 0, stream>>>(target, draft, tokens, uniforms, kd,
                                                               v, chunks, ws, out_tokens, out_num,
                                                               flags);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  wsum_kernel<<<dim3((unsigned)chunks, (unsigned)b), dim3(kThreads), 0, stream>>>(target, draft, kd,
                                                                                  v, chunks, ws);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  sample_kernel<<<dim3((unsigned)b), dim3(kThreads), 0, stream>>>(target, draft, uniforms, kd, v,
                                                                  chunks, ws, out_tokens, flags);
  return hipGetLastError();
}

}  // namespace mxs
