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
//   decide  grid (pieces, sequences), 1024-logit pieces: every workgroup
//           combines its sequence's chunk statistics into (max, sum) per row,
//           forms p_i(x_i) and q_i(x_i) in fp64 from the logits the stats
//           kernel gathered (one lane per draft position), takes n = first
//           rejection with a ballot, then sums the final weights w (residual
//           or bonus row) over its own piece. Piece 0 writes the decisions.
//   sample  one workgroup per sequence: a block scan of the piece totals
//           finds the piece holding u_K·Z; its weights are recomputed exactly
//           as decide computed them, a block scan of the thread totals finds
//           the thread, and that thread's 4 weights give t*.
// With sampling transforms (spec_accept_sampled) two or four selection kernels
// run first and leave one order-key threshold per row (top-k / top-p, see "top-k /
// top-p thresholds" below); the three kernels then read the transformed laws.
// The fp64 exponentials bound decide and sample at small batches, so their
// pieces are small: many workgroups share the work of one sequence.
// All probabilities and prefix sums are fp64; the result can differ from an
// exact-arithmetic draw only when u_K·Z lies within ~1e-15·Z of an interval
// end. Rounding guards: if no crossing is found where the level above
// placed it, the last positive-weight token of that range is taken, so a
// zero-weight token is never returned.
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "internal.hpp"

// No FMA contraction: p - q with p = e_t/S_t must be exactly 0 when the target
// and draft rows are equal, and the decide and sample kernels must compute
// bit-identical weights.
#pragma clang fp contract(off)

namespace mxs {
namespace {

// stats: 256 threads x 16 logits per 4096-logit chunk. decide / sample: 256
// threads x 4 logits per 1024-logit piece; both walk the same pieces, so the
// piece totals of the final weights written by decide are the ones sample scans.
constexpr int kThreads = 256;
constexpr int kPer = 16;
constexpr int kChunk = kThreads * kPer;  // 4096 logits per chunk
constexpr int kWThreads = 256;
constexpr int kWPer = 4;                   // logits per thread in decide / sample
constexpr int kPiece = kWThreads * kWPer;  // 1024 logits per piece
constexpr int kPassBatch = 3;              // statistics passes whose loads decide keeps in flight
constexpr int kMaxRows = 65;               // 2 * 32 + 1 rows per sequence
constexpr int kQuadChunks = 8;             // chunks per thread when a quad combines a row


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
  float* gz;       // [rows] logit of the row's draft token (written by the chunk holding it)
  struct Decision* dec;  // [b] n and the statistics of the final draw's rows
  double* zres;    // [b][pieces] piece totals of the final weights
  double* zp;      // [b][pieces] piece totals of p_n (zero-residual fallback)
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  size_t cmax, csum, cbad, gz, dec, zres, zp;
  // sampling transforms only
  size_t thr, selcnt, selmass, selstate, selarrive, selrkey, selcandn, selcand, selrbad, sdone;
  size_t total;
};

struct SelState;

inline Layout layout(int64_t b, int64_t kd, int64_t v, bool sampled = false) {
  const int64_t rows = b * (2 * kd + 1);
  const int64_t chunks = (v + kChunk - 1) / kChunk;
  const int64_t pieces = (v + kPiece - 1) / kPiece;
  Layout L;
  size_t off = 0;
  L.cmax = off;
  off = align256(off + sizeof(float) * rows * chunks);
  L.csum = off;
  off = align256(off + sizeof(double) * rows * chunks);
  L.cbad = off;
  off = align256(off + sizeof(int32_t) * rows * chunks);
  L.gz = off;
  off = align256(off + sizeof(float) * rows);
  L.dec = off;
  off = align256(off + sizeof(Decision) * b);
  L.zres = off;
  off = align256(off + sizeof(double) * b * pieces);
  L.zp = off;
  off = align256(off + sizeof(double) * b * pieces);
  if (sampled) {
    constexpr size_t kBuckets = 4096, kStateBytes = 48, kCandKeys = 8192;
    L.thr = off;
    off = align256(off + sizeof(uint32_t) * rows);
    L.selcnt = off;
    off = align256(off + sizeof(uint32_t) * rows * kBuckets);
    L.selmass = off;
    off = align256(off + sizeof(double) * rows * kBuckets);
    L.selstate = off;
    off = align256(off + kStateBytes * rows);
    L.selarrive = off;
    off = align256(off + sizeof(uint32_t) * rows);
    L.selrkey = off;
    off = align256(off + sizeof(uint32_t) * rows);
    L.selcandn = off;
    off = align256(off + sizeof(uint32_t) * rows);
    L.selcand = off;
    off = align256(off + sizeof(uint32_t) * rows * kCandKeys);
    L.selrbad = off;
    off = align256(off + sizeof(uint32_t) * rows);
    L.sdone = off;
    off = align256(off + sizeof(uint32_t) * rows);
  }
  L.total = off;
  return L;
}

// Logit row j of sequence s: rows 0..kd are target rows, kd+1..2kd draft rows.
__device__ inline const float* row_ptr(const float* target, const float* draft, int64_t s, int kd,
                                       int j, int64_t v) {
  if (j <= kd) return target + ((size_t)s * (kd + 1) + j) * (size_t)v;
  return draft + ((size_t)s * kd + (j - kd - 1)) * (size_t)v;
}

// ---------------------------------------------------------------- sampling transforms
// Temperature, grammar mask and top-k / top-p thresholds, applied to every target
// and draft row alike. A token of row j is live iff its mask bit (mask row j for
// target rows, j - kd - 1 for draft rows: one mask per position) is set and the
// order key of its logit is at least the row's threshold. A removed token's logit
// is replaced by -inf before any exponential, so it has probability 0; exponents
// are (z - max) / tau.
struct Transform {
  const uint32_t* mask;  // [b][kd+1][words] bits, 1 = allowed; or null
  const uint32_t* thr;   // [rows] order-key thresholds; or null (no top-k / top-p)
  double inv_tau;        // 1 / temperature
  int words;             // ceil(v / 32)
  const uint32_t* sdone; // [rows] 1: the row's statistics were written by the selection; or null
};

// fp32 -> uint32 with the same order (negatives reversed below the positives; -0 and
// +0 compare equal as logits, so they get one key).
__device__ inline uint32_t order_key(float z) {
  const uint32_t b = __float_as_uint(z == 0.0f ? 0.0f : z);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ inline int mask_row(int j, int kd) { return j <= kd ? j : j - kd - 1; }

// Mask words of mask row mi of sequence s (null without a mask).
__device__ inline const uint32_t* mask_words(const Transform& tr, int64_t s, int kd, int mi) {
  return tr.mask ? tr.mask + ((size_t)s * (kd + 1) + mi) * (size_t)tr.words : nullptr;
}

__device__ inline float live_logit(float z, int t, const uint32_t* words, uint32_t thr) {
  const bool allowed = words ? ((words[t >> 5] >> (t & 31)) & 1u) != 0u : true;
  return (allowed && order_key(z) >= thr) ? z : -INFINITY;
}

// ---------------------------------------------------------------- stats
// kT: the transformed laws (mask, threshold and temperature from tr).
template <bool kVec4, bool kT>
__global__ __launch_bounds__(kThreads) void stats_kernel(const float* __restrict__ target,
                                                         const float* __restrict__ draft,
                                                         const int32_t* __restrict__ tokens, int kd,
                                                         int v, int chunks, Workspace ws,
                                                         Transform tr) {
  __shared__ double lds_d[kThreads / kWave];
  __shared__ float lds_f[kThreads / kWave];
  __shared__ int lds_i[kThreads / kWave];
  __shared__ double tab[32];  // 2^(j/32) for the table-driven exp (visible after block_max)
  if (threadIdx.x < 32) tab[threadIdx.x] = kExp2Table32[threadIdx.x];
  const int64_t rowg = blockIdx.x;  // row index over all sequences
  if constexpr (kT) {
    if (tr.sdone && tr.sdone[rowg]) return;  // written by the selection (uniform per workgroup)
  }
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
  // the logit of this row's draft token x (target row i < kd or draft row i), if it is in this
  // chunk: thread 0 loads it (and its mask word) with the chunk and stores it at the end
  int xi = -1;
  if (j < kd) xi = tokens[(size_t)s * kd + j];
  else if (j > kd) xi = tokens[(size_t)s * kd + (j - kd - 1)];
  const bool x_here = xi >= base && xi < base + kChunk;  // uniform
  float mx = -INFINITY;
  int bad = 0;
  const uint32_t* mw = nullptr;
  uint32_t thr = 0u;
  if constexpr (kT) {
    mw = mask_words(tr, s, kd, mask_row(j, kd));
    thr = tr.thr ? tr.thr[rowg] : 0u;
  }
  float zx = -INFINITY;     // past the row: -inf, as the chunk's own padding
  uint32_t xword = ~0u;
  if (x_here && threadIdx.x == 0 && xi < v) {
    zx = z[xi];
    if (kT && mw) xword = mw[xi >> 5];
  }
  // mask words: one per 4 tokens on the vector path; the word index is clamped into the
  // row (tokens past v are already -inf)
  uint32_t words[kPer];
  if constexpr (kT) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = kVec4 ? base + 4 * (threadIdx.x + kThreads * (q / 4)) : base + threadIdx.x + kThreads * q;
      if (!kVec4 || q % 4 == 0) words[q] = mw ? mw[(e < v ? e : v - 1) >> 5] : 0xFFFFFFFFu;
      else words[q] = words[q - q % 4];
    }
  }
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    bad |= (int)nan_or_pinf(vals[q]);
    const int e = kVec4 ? base + 4 * (threadIdx.x + kThreads * (q / 4)) + (q % 4)
                        : base + threadIdx.x + kThreads * q;
    if constexpr (kT) {
      const bool ok = ((words[q] >> (e & 31)) & 1u) && order_key(vals[q]) >= thr;
      vals[q] = ok ? vals[q] : -INFINITY;
    }
    mx = fmaxf(mx, vals[q]);
  }
  if (x_here && threadIdx.x == 0) {
    if constexpr (kT) zx = (((xword >> (xi & 31)) & 1u) && order_key(zx) >= thr) ? zx : -INFINITY;
    ws.gz[rowg] = zx;
  }
  block_max_or<kThreads>(mx, bad, lds_f, lds_i);
  double acc = 0.0;
  if (mx != -INFINITY && !bad) {
    const double m64 = (double)mx;
    const ExpK ek = exp_consts();
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      if constexpr (kT) acc += exp_neg_f64_tab(((double)vals[q] - m64) * tr.inv_tau, tab, ek);
      else acc += exp_neg_f64_tab((double)vals[q] - m64, tab, ek);
    }
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
  const double* tab;  // kExp2Table32 in LDS, for exp_neg_f64_tab
  ExpK ek;            // its constants, in registers
  const float* zt;
  const float* zd;  // nullptr for the bonus row
  double mt, inv_st, md, inv_sd;
  // transformed laws only: 1/tau, the rows' thresholds and the position's mask words
  double inv_tau;
  uint32_t thr_t, thr_d;
  const uint32_t* mw;
};

// Final weights and p_n of kWPer consecutive tokens from their logits zt, zd (removed
// tokens already -inf when kT).
template <bool kT>
__device__ inline void weights_from(const FinalRows& fr, const float (&zt)[kWPer],
                                    const float (&zd)[kWPer], double (&wf)[kWPer],
                                    double (&wp)[kWPer]) {
#pragma unroll
  for (int j = 0; j < kWPer; ++j) {
    const double dt = kT ? ((double)zt[j] - fr.mt) * fr.inv_tau : (double)zt[j] - fr.mt;
    const double p = exp_neg_f64_tab(dt, fr.tab, fr.ek) * fr.inv_st;
    wp[j] = p;
    if (fr.zd) {
      const double dd = kT ? ((double)zd[j] - fr.md) * fr.inv_tau : (double)zd[j] - fr.md;
      const double q = exp_neg_f64_tab(dd, fr.tab, fr.ek) * fr.inv_sd;
      const double d = p - q;
      wf[j] = d > 0.0 ? d : 0.0;
    } else {
      wf[j] = p;
    }
  }
}

// Final weights and p_n of the kWPer consecutive tokens t0 .. t0+kWPer-1 (zero past v).
// Both rows are loaded before any arithmetic (one 16-byte load each when aligned).
template <bool kT>
__device__ inline void thread_weights(const FinalRows& fr, int t0, int v, bool vec4,
                                      double (&wf)[kWPer], double (&wp)[kWPer]) {
  float zt[kWPer], zd[kWPer];
  if (vec4 && t0 + kWPer <= v) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(fr.zt + t0);
    f32x4 b = a;
    if (fr.zd) b = *reinterpret_cast<const f32x4*>(fr.zd + t0);
#pragma unroll
    for (int j = 0; j < kWPer; ++j) {
      zt[j] = a[j];
      zd[j] = b[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kWPer; ++j) {
      const bool in = t0 + j < v;
      zt[j] = in ? fr.zt[t0 + j] : -INFINITY;
      zd[j] = (in && fr.zd) ? fr.zd[t0 + j] : -INFINITY;
    }
  }
  if constexpr (kT) {
#pragma unroll
    for (int j = 0; j < kWPer; ++j) {
      if (t0 + j < v) {
        zt[j] = live_logit(zt[j], t0 + j, fr.mw, fr.thr_t);
        zd[j] = live_logit(zd[j], t0 + j, fr.mw, fr.thr_d);
      }
    }
  }
  weights_from<kT>(fr, zt, zd, wf, wp);
}

// ---------------------------------------------------------------- final draw
constexpr int kNone = 0x7fffffff;

// The final token of sequence s by inverse CDF, in two levels that every thread
// of the workgroup enters. select_piece scans the piece totals written by the
// decide workgroups of the sequence and picks the piece holding u_K·Z;
// select_token scans the thread totals of that piece's final weights (computed
// exactly as its decide workgroup computed them: same code, same summation
// order, so the running totals inside the piece add up to its stored total),
// picks the thread, and that thread's 4 weights give the token.
struct PieceChoice {
  int c;        // chosen piece, or -1 when no piece has positive weight
  bool found;   // u_K·Z crossed a running total (otherwise c is the last positive piece)
  bool use_p;   // zero residual mass: the draw is from p_n
  double base;  // running total before piece c
  double uz;    // u_K·Z
};

constexpr int kWWaves = kWThreads / kWave;

// Over the workgroup, index base + threadIdx.x: the first index whose thread has
// first_cond (kNone if none) and the last whose thread has last_cond (-1 if none).
// One ballot per wave and the per-wave answers through LDS (lds: 2 * kWWaves
// ints); the barriers inside also publish LDS writes made before the call.
__device__ inline int2 block_first_last(bool first_cond, bool last_cond, int base, int* lds) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const unsigned long long m1 = __ballot(first_cond);
  const unsigned long long m2 = __ballot(last_cond);
  if (lane == 0) {
    lds[w] = m1 ? base + w * kWave + __builtin_ctzll(m1) : kNone;
    lds[kWWaves + w] = m2 ? base + w * kWave + 63 - __builtin_clzll(m2) : -1;
  }
  __syncthreads();
  int2 r = make_int2(kNone, -1);
#pragma unroll
  for (int i = 0; i < kWWaves; ++i) {
    r.x = min(r.x, lds[i]);
    r.y = max(r.y, lds[kWWaves + i]);
  }
  __syncthreads();
  return r;
}

// zres0 / zp0: this thread's piece totals, loaded by the caller when
// pieces <= kWThreads; u_last: the sequence's final uniform u_K. Loading them at
// kernel entry keeps global loads from waiting behind the block barriers here.
// flags may be null (the zero-residual flag is then left to another workgroup).
__device__ PieceChoice select_piece(int n, int kd, int pieces, int64_t s, const Workspace& ws,
                                    float u_last, int32_t* __restrict__ flags, double zres0,
                                    double zp0, double* lds_scan, double* s_incl, int* s_fl) {
  const int tid = threadIdx.x;
  PieceChoice pc;
  pc.use_p = false;
  pc.base = 0.0;
  double Z = 0.0;
  int c = kNone, last = -1;
  if (pieces <= kWThreads) {
    // one piece per thread: both totals loaded once, one scan (two on the zero-residual path)
    double incl = block_inclusive_scan_f64<kWThreads>(zres0, lds_scan);
    if (tid == kWThreads - 1) s_incl[0] = incl;
    __syncthreads();
    Z = s_incl[0];
    double zc = zres0;
    __syncthreads();
    if (!(Z > 0.0)) {  // zero residual mass (rounding): draw from p_n instead
      pc.use_p = true;
      zc = zp0;
      incl = block_inclusive_scan_f64<kWThreads>(zp0, lds_scan);
      if (tid == kWThreads - 1) s_incl[0] = incl;
      __syncthreads();
      Z = s_incl[0];
      __syncthreads();
      if (n < kd && tid == 0) raise_flag(flags, MXS_FLAG_RESIDUAL_ZERO);
    }
    const double uz = (double)u_last * Z;
    s_incl[tid] = incl;
    const bool pos = tid < pieces && zc > 0.0;
    const int2 fl = block_first_last(pos && uz < incl, pos, 0, s_fl);
    c = fl.x;
    last = fl.y;
    if (c != kNone) pc.base = c > 0 ? s_incl[c - 1] : 0.0;
  } else {
    // many pieces: rounds of kWThreads piece totals with a carry
    const double* zr = ws.zres + s * pieces;
    for (int pass = 0; pass < 2; ++pass) {
      double carry = 0.0;
      for (int c0 = 0; c0 < pieces; c0 += kWThreads) {
        const int cc = c0 + tid;
        const double incl =
            carry + block_inclusive_scan_f64<kWThreads>(cc < pieces ? zr[cc] : 0.0, lds_scan);
        if (tid == kWThreads - 1) s_incl[0] = incl;
        __syncthreads();
        carry = s_incl[0];
        __syncthreads();
      }
      Z = carry;
      if (Z > 0.0 || pass == 1) break;
      pc.use_p = true;
      zr = ws.zp + s * pieces;
      if (n < kd && tid == 0) raise_flag(flags, MXS_FLAG_RESIDUAL_ZERO);
    }
    const double uz = (double)u_last * Z;
    double carry = 0.0;
    for (int c0 = 0; c0 < pieces; c0 += kWThreads) {
      const int cc = c0 + tid;
      const double zc = cc < pieces ? zr[cc] : 0.0;
      const double incl = carry + block_inclusive_scan_f64<kWThreads>(zc, lds_scan);
      s_incl[tid] = incl;
      const bool pos = cc < pieces && zc > 0.0;
      const int2 fl = block_first_last(pos && uz < incl, pos, c0, s_fl);
      last = max(last, fl.y);
      if (fl.x != kNone) {
        c = fl.x;
        pc.base = c > c0 ? s_incl[c - c0 - 1] : carry;
        break;
      }
      carry = s_incl[kWThreads - 1];
      __syncthreads();
    }
  }
  pc.uz = (double)u_last * Z;
  pc.found = c != kNone;
  // no crossing (u >= 1 or rounding): the last piece with positive weight (-1 if none;
  // a valid row always has positive mass)
  pc.c = pc.found ? c : last;
  __syncthreads();
  return pc;
}

// Level 2 and 3 inside piece pc.c; wf / wp are this thread's 4 weights of that
// piece (tokens t0 .. t0+3). The thread that owns the token writes it.
__device__ void select_token(const PieceChoice& pc, int n, int kd, int64_t s, int t0,
                             const double (&wf)[kWPer], const double (&wp)[kWPer],
                             int32_t* __restrict__ out_tokens, double* lds_scan, double* s_incl,
                             int* s_fl) {
  const int tid = threadIdx.x;
  double tau = 0.0;
#pragma unroll
  for (int j = 0; j < kWPer; ++j) tau += pc.use_p ? wp[j] : wf[j];
  const double sincl = block_inclusive_scan_f64<kWThreads>(tau, lds_scan);
  s_incl[tid] = sincl;
  const bool pos = tau > 0.0;
  const int2 fl = block_first_last(pos && pc.found && pc.uz < pc.base + sincl, pos, 0, s_fl);
  // the crossing thread, or (fallback piece / rounding) the last thread with positive weight
  const int ti = fl.x != kNone ? fl.x : fl.y;
  if (tid != ti) return;
  // ---- level 3: the 4 tokens of thread ti (its weights are already in registers)
  const double before = pc.base + (ti > 0 ? s_incl[ti - 1] : 0.0);
  double run = 0.0;
  int pick = -1, lastpos = -1;
#pragma unroll
  for (int j = 0; j < kWPer; ++j) {
    const double w = pc.use_p ? wp[j] : wf[j];
    run += w;
    if (w > 0.0) lastpos = t0 + j;
    if (pc.found && pick < 0 && w > 0.0 && pc.uz < before + run) pick = t0 + j;
  }
  out_tokens[(size_t)s * (kd + 1) + n] = pick >= 0 ? pick : lastpos;
}

// The whole draw for one sequence by one workgroup (the sample kernel).
template <bool kT>
__device__ void draw_final(const FinalRows& fr, int n, int kd, int v, int pieces, int64_t s,
                           const Workspace& ws, float u_last,
                           int32_t* __restrict__ out_tokens, int32_t* __restrict__ flags, int vec4,
                           double zres0, double zp0, double* lds_scan, double* s_incl,
                           int* s_fl) {
  const PieceChoice pc = select_piece(n, kd, pieces, s, ws, u_last, flags, zres0, zp0, lds_scan,
                                      s_incl, s_fl);
  if (pc.c < 0) return;
  const int t0 = pc.c * kPiece + (int)threadIdx.x * kWPer;
  double wf[kWPer], wp[kWPer];
  thread_weights<kT>(fr, t0, v, vec4, wf, wp);
  select_token(pc, n, kd, s, t0, wf, wp, out_tokens, lds_scan, s_incl, s_fl);
}

// ---------------------------------------------------------------- top-k / top-p thresholds
// A row's threshold is an order key: a token stays iff it is allowed, finite and its key
// is at least the threshold (0 keeps every allowed finite token). The key splits into
// digit 0 (its top 12 bits: sign, exponent and 3 fraction bits of the logit) and two
// 10-bit digits. Top-k with k at most 256 and at least 2k list slots per chunk (every
// common vocabulary) takes two kernels:
//   sel_chunk     grid (rows, chunks), one read of the logits: each chunk's keys from a lower
//                 bound of its own k-th largest up go to the chunk's own (interleaved) slots of
//                 the row's list (see sel_chunk below), with a record of their count and bound.
//   sel_finish    the union of the chunks' candidates from the largest bound up, cut by the
//                 k-th largest of its threads' maxima; at most 64 left (the usual case) are
//                 finished by one wave without a barrier (sort, thresholds, row statistics),
//                 more as below.
// Top-p alone and larger k take four:
//   sel_clear     zeroes each row's digit-0 histogram, counters and maximum.
//   sel_count     grid (rows, groups of 4096-logit chunks), one read of the logits: the row
//                 maximum (an atomic max of order keys), whether the row holds a NaN or +inf,
//                 and the digit-0 histogram: counts for top-k; for top-p alone masses
//                 exp(z / tau) against the reference 0, which needs no row maximum. The row's
//                 last workgroup to arrive finds the digit-0 bucket holding the boundary (the
//                 lowest non-empty bucket with fewer than k tokens, or less than P·S mass,
//                 strictly above it) and sets the row's course (SelMode).
//   sel_collect   grid (rows, chunks), one read: the candidate keys into the row's list — for
//                 top-k every key from the boundary bucket up (fewer than k + the bucket's
//                 count), for top-p the boundary bucket's keys.
//   sel_finish    one workgroup per row, candidates in LDS: a list of up to kSortMax keys is
//                 sorted (descending) and the thresholds read off it — top-k is the k-th key;
//                 top-p tests each distinct key's strictly-larger mass, summed in the sorted
//                 order — and for top-k the row's statistics are written too (the stats kernel
//                 then skips the row). A longer top-k list is first cut to the keys from a
//                 lower bound of its k-th largest up (the k-th largest of the threads' maxima
//                 over it), then, if still longer, resolved by radix passes over the keys in LDS
//                 and cut to the kept set; top-p lists likewise by radix passes. A row whose
//                 candidates do not fit the list, a top-p row whose top-k kept every token, and
//                 a top-p row whose exp(z / tau) would leave fp64's range against 0 are finished
//                 by this workgroup alone with radix passes over the row (histograms in LDS,
//                 masses against the row maximum).
// The digit-0 histograms are added with device-scope atomics; each workgroup waits for its
// own before it counts its arrival, and the resolving workgroup reads them with device-scope
// loads: no plain store is shared between workgroups of one launch.
constexpr int kSelBits0 = 12;
constexpr int kSelB0 = 1 << kSelBits0;      // digit-0 buckets
constexpr int kSelShift0 = 32 - kSelBits0;  // digit 0 = key >> 20
constexpr int kSelBits1 = 10;               // digits 1 and 2
constexpr int kCandLog2 = 13;
constexpr int kCand = 1 << kCandLog2;       // candidate keys per row
constexpr int kFThreads = 512;              // sel_finish
constexpr int kFWaves = kFThreads / kWave;
constexpr int kSortMax = 512;  // candidate lists up to this size are sorted (fixed-order sums)
static_assert(kSortMax <= kFThreads, "a sorted list is walked with one candidate per thread");
// top-p alone takes its digit-0 masses against the reference 0 when the row maximum m has
// m / tau in this range: every exp(z / tau) and their sum stay finite, and a token that
// underflows against 0 has mass below e^-45 of the maximum's (it cannot sit at a boundary
// that P < 1 - 2^-24 places among at most 2^26 tokens).
constexpr double kRef0Lo = -650.0, kRef0Hi = 690.0;

enum SelMode : uint32_t {
  kSelDone = 0,       // threshold known: state.thr
  kSelCompactK = 1,   // candidates: every key >= state.lo (top-k, then top-p on them)
  kSelCompactP = 2,   // candidates: the keys of digit-0 bucket state.lo (top-p)
  kSelSlowK = 3,      // top-k continues in digit-0 bucket state.lo by sel_finish's radix passes
  kSelSlowP = 4,      // top-p likewise
  kSelSlowPFull = 5,  // top-p over every allowed token by sel_finish's radix passes
  kSelSlowKFull = 6,  // top-k (then top-p) over every allowed token by sel_finish's radix passes
};

struct SelState {
  uint32_t mode;   // SelMode
  uint32_t lo;     // kSelCompactK: lowest candidate key; else the boundary's digit-0 bucket
  uint32_t thr;    // kSelDone: the threshold
  uint32_t pad;
  double carry;    // count (top-k) or mass (top-p) strictly above the bucket
  double s1;       // top-p: S, the mass of the tokens top-k left
  float rmax;      // largest allowed finite logit (the mass reference)
  uint32_t pad2[3];
};
static_assert(sizeof(SelState) == 48, "workspace layout assumes a 48-byte selection state");

struct SelBufs {
  uint32_t* cnt;     // [rows][kSelB0] digit-0 counts
  double* mass;      // [rows][kSelB0] digit-0 masses
  SelState* state;   // [rows]
  uint32_t* arrive;  // [rows] workgroups of the current launch that have finished
  uint32_t* rkey;    // [rows] order key of the row maximum (0: no allowed finite logit)
  uint32_t* candn;   // [rows] candidate keys collected
  uint32_t* cand;    // [rows][kCand]
  uint32_t* thr;     // [rows] the thresholds
  uint32_t* rbad;    // [rows] a NaN or +inf seen in the row (sel_count)
};

// spec_accept_sampled only: sel_finish writes the stats kernel's outputs for rows whose kept
// set it holds sorted (top-k candidates, at most kSortMax) and marks them in sdone, so the
// stats kernel skips them; null for the threshold-only entry point.
struct SelStats {
  float* cmax;            // [rows][chunks]
  double* csum;           // [rows][chunks]
  int32_t* cbad;          // [rows][chunks]
  float* gz;              // [rows]
  uint32_t* sdone;        // [rows] 1: statistics written here
  const int32_t* tokens;  // [b][kd] draft tokens
  int chunks;
};

// The logit of a row's draft token for the statistics the selection writes (the stats kernel's
// gz), loaded by one thread early in the finishing workgroup so that its two dependent loads (the
// token, then its logit and mask word) are not at the end of the workgroup's life.
struct DraftLogit {
  int xi = -1;          // the token; -1: the bonus row, no statistics, or a token outside [0, v)
  float zx = 0.0f;      // its logit
  uint32_t word = ~0u;  // its mask word (all ones without a mask)

  __device__ void load_token(const SelStats& ss, int64_t s, int j, int kd, int v) {
    if (!ss.cmax) return;
    if (j < kd) xi = ss.tokens[(size_t)s * kd + j];
    else if (j > kd) xi = ss.tokens[(size_t)s * kd + (j - kd - 1)];
    if (xi >= v) xi = -1;
  }
  __device__ void load_logit(const float* __restrict__ z, const uint32_t* mw) {
    if (xi < 0) return;
    zx = z[xi];
    if (mw) word = mw[xi >> 5];
  }
  // gz: the logit if the token is allowed and kept (key >= thr), else -inf
  __device__ void put(const SelStats& ss, int64_t rowg, uint32_t thr) const {
    if (xi < 0) return;
    const bool allowed = ((word >> (xi & 31)) & 1u) != 0u;
    ss.gz[rowg] = (allowed && order_key(zx) >= thr) ? zx : -INFINITY;
  }
};

struct SelArgs {
  int top_k;      // 0: off
  double top_p;   // >= 1: off
  int chunks;     // 4096-logit chunks per row
  int slot_log2;  // > 0: top-k by per-chunk candidates (sel_chunk), 2^slot_log2 per chunk: candidate
                  // i of chunk c at list position i·2^chunk_log2 + c
  int chunk_log2; // 2^chunk_log2 >= chunks (with slot_log2: the list's first 2^(sum) keys)
};

// The logit of an order key (inverse of order_key; -0 comes back as +0).
__device__ inline float key_logit(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// The allowed logits of this thread's 16 tokens of a chunk (removed ones: NaN), in the
// stats kernel's order.
// *bad is ORed with 1 when a token of the chunk (allowed or not) is NaN or +inf.
// Every load is issued before any is used (an index past the row reads the row's first element,
// which is then discarded), so a workgroup waits for one memory trip, not one per load.
template <bool kVec4>
__device__ inline void chunk_logits(const float* __restrict__ z, const uint32_t* mw, int base, int v,
                                    float (&vals)[kPer], int* bad = nullptr) {
  int b = 0;
  if constexpr (kVec4) {
    constexpr int kV = kPer / 4;
    f32x4 t[kV];
    uint32_t w[kV];
#pragma unroll
    for (int q = 0; q < kV; ++q) {
      const int e = base + 4 * ((int)threadIdx.x + kThreads * q);
      t[q] = *reinterpret_cast<const f32x4*>(z + (e < v ? e : 0));
    }
    if (mw) {
#pragma unroll
      for (int q = 0; q < kV; ++q) {
        const int e = base + 4 * ((int)threadIdx.x + kThreads * q);
        w[q] = mw[(e < v ? e : 0) >> 5];  // the 4 tokens share one mask word
      }
    } else {
#pragma unroll
      for (int q = 0; q < kV; ++q) w[q] = 0xFFFFFFFFu;
    }
#pragma unroll
    for (int q = 0; q < kV; ++q) {
      const int e = base + 4 * ((int)threadIdx.x + kThreads * q);
      const bool in = e < v;  // v % 4 == 0: the whole vector or none of it
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = t[q][i];
        const uint32_t fin = __builtin_isfinite(x) ? 1u : 0u;
        b |= (int)(in & nan_or_pinf(x));
        const uint32_t ok = (uint32_t)in & (w[q] >> ((e + i) & 31)) & fin;
        vals[4 * q + i] = ok ? x : NAN;
      }
    }
  } else {
    float t[kPer];
    uint32_t w[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = base + (int)threadIdx.x + kThreads * q;
      t[q] = z[e < v ? e : 0];
    }
    if (mw) {
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int e = base + (int)threadIdx.x + kThreads * q;
        w[q] = mw[(e < v ? e : 0) >> 5];
      }
    } else {
#pragma unroll
      for (int q = 0; q < kPer; ++q) w[q] = 0xFFFFFFFFu;
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = base + (int)threadIdx.x + kThreads * q;
      const bool in = e < v;
      const float x = t[q];
      const uint32_t fin = __builtin_isfinite(x) ? 1u : 0u;
      b |= (int)(in & nan_or_pinf(x));
      const uint32_t ok = (uint32_t)in & (w[q] >> (e & 31)) & fin;
      vals[q] = ok ? x : NAN;
    }
  }
  if (bad) *bad |= b;
}

// Block-wide max of one int per thread (kT threads); lds: kT / kWave ints.
template <int kT>
__device__ inline int block_max_i32(int v, int* lds) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v = max(v, __shfl_xor(v, o));
  if ((threadIdx.x & (kWave - 1)) == 0) lds[threadIdx.x / kWave] = v;
  __syncthreads();
  int r = lds[0];
#pragma unroll
  for (int i = 1; i < kT / kWave; ++i) r = max(r, lds[i]);
  __syncthreads();
  return r;
}

// The boundary bucket of one histogram walked from the largest key down. Thread t holds
// buckets nb - 1 - (t·kPB + i), i < kPB (kT·kPB = nb): counts c and weights w (counts
// for top-k, masses for top-p). Returns the lowest non-empty bucket whose weight strictly
// above it, plus carry, is below target (-1: none) with that sum in *above, and the sum of
// all weights in *total. Every thread returns the same values. lds: kT / kWave doubles,
// s_d: 2 doubles, s_i: kT / kWave ints.
template <int kT, int kPB>
__device__ int resolve_desc(const uint32_t (&c)[kPB], const double (&w)[kPB], double carry, double target,
                            double* above, double* total, double* lds, double* s_d, int* s_i) {
  const int tid = threadIdx.x;
  double local = 0.0;
#pragma unroll
  for (int i = 0; i < kPB; ++i) local += w[i];
  const double incl = block_inclusive_scan_f64<kT>(local, lds);
  if (tid == kT - 1) s_d[1] = incl;
  double run = carry + (incl - local);
  int best = -1;
  double best_above = 0.0;
#pragma unroll
  for (int i = 0; i < kPB; ++i) {
    if (run < target && c[i] > 0u) {
      best = tid * kPB + i;
      best_above = run;
    }
    run += w[i];
  }
  // descending positions grow with the thread index: the largest qualifying position is the
  // lowest qualifying bucket
  const int b = block_max_i32<kT>(best, s_i);  // its barrier orders s_d[1] too
  if (b >= 0 && best == b) s_d[0] = best_above;
  __syncthreads();
  *above = b >= 0 ? s_d[0] : 0.0;
  *total = s_d[1];
  __syncthreads();
  return b >= 0 ? kT * kPB - 1 - b : -1;
}

// Zeroes the row's digit-0 histogram (counts, or with `mass` the masses), arrival count,
// candidate count and maximum.
__global__ __launch_bounds__(kThreads) void sel_clear_kernel(SelBufs sb, int mass) {
  const int64_t row = blockIdx.x;
  if (!mass) {
    u32x4* c = reinterpret_cast<u32x4*>(sb.cnt + row * kSelB0);
    for (int i = threadIdx.x; i < kSelB0 / 4; i += kThreads) c[i] = u32x4{0u, 0u, 0u, 0u};
  } else {
    u32x4* m = reinterpret_cast<u32x4*>(sb.mass + row * kSelB0);
    for (int i = threadIdx.x; i < kSelB0 / 2; i += kThreads) m[i] = u32x4{0u, 0u, 0u, 0u};
  }
  if (threadIdx.x == 0) {
    sb.arrive[row] = 0u;
    sb.candn[row] = 0u;
    sb.rkey[row] = 0u;
    sb.rbad[row] = 0u;
  }
}

// This workgroup's histogram (in LDS: counts, or with kMass masses) added into the row's;
// then its arrival. Returns true in the row's last workgroup to arrive.
template <bool kMass>
__device__ bool flush_and_arrive(const uint32_t* hc, const double* hm, uint32_t* gc, double* gm,
                                 uint32_t* arrive, int wgs, int* s_last) {
  __syncthreads();
  for (int b = threadIdx.x; b < kSelB0; b += kThreads) {
    if constexpr (kMass) {
      if (hm[b] != 0.0) atomicAdd(&gm[b], hm[b]);
    } else {
      if (hc[b] != 0u) atomicAdd(&gc[b], hc[b]);
    }
  }
  // the additions (and the maximum) are device-scope atomics performed in L2; each wave
  // waits until its own have completed, so the count cannot run ahead of them
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t before = __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_last = before == (uint32_t)(wgs - 1);
  }
  __syncthreads();
  return *s_last != 0;
}

// Thread t's 16 digit-0 buckets of the row histogram, largest keys first (device-scope loads:
// other workgroups of this launch added them): counts, or with kMass masses (a bucket is
// non-empty when its mass is positive).
template <bool kMass>
__device__ inline void load_desc16(const uint32_t* gc, const double* gm, uint32_t (&c)[16], double (&w)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int b = kSelB0 - 1 - ((int)threadIdx.x * 16 + i);
    if constexpr (kMass) {
      w[i] = __hip_atomic_load(&gm[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      c[i] = w[i] > 0.0 ? 1u : 0u;
    } else {
      c[i] = __hip_atomic_load(&gc[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      w[i] = (double)c[i];
    }
  }
}

// kMass: top-p alone, the digit-0 masses exp(z / tau) against the reference 0 (a token whose
// mass underflows there is below e^-45 of the maximum's and is never kept). Else top-k, the
// digit-0 counts. A workgroup takes chunks [blockIdx.y · cpw, + cpw) of its row (several chunks
// per workgroup at large batches: fewer histograms to add into the row's).
template <bool kVec4, bool kMass>
__global__ __launch_bounds__(kThreads) void sel_count_kernel(const float* __restrict__ target,
                                                             const float* __restrict__ draft, int kd,
                                                             int v, int chunks, int cpw, Transform tr,
                                                             SelBufs sb, SelArgs sa) {
  __shared__ uint32_t hc[kMass ? 1 : kSelB0];
  __shared__ double hm[kMass ? kSelB0 : 1];
  __shared__ double tab[32];
  __shared__ float lds_f[kThreads / kWave];
  __shared__ double lds_scan[kThreads / kWave];
  __shared__ double s_d[2];
  __shared__ int s_i[kThreads / kWave];
  __shared__ int s_last;
  const int64_t rowg = blockIdx.x;
  const int per_seq = 2 * kd + 1;
  const int64_t s = rowg / per_seq;
  const int j = (int)(rowg % per_seq);
  const int tid = threadIdx.x;
  if (kMass && tid < 32) tab[tid] = kExp2Table32[tid];
  for (int b = tid; b < kSelB0; b += kThreads) {
    if constexpr (kMass) hm[b] = 0.0;
    else hc[b] = 0u;
  }
  const float* zrow = row_ptr(target, draft, s, kd, j, v);
  const uint32_t* mw = mask_words(tr, s, kd, mask_row(j, kd));
  float mx = -INFINITY;
  const int c0 = (int)blockIdx.y * cpw, c1 = min(chunks, c0 + cpw);
  int bad = 0;
  ExpK ek{};
  if constexpr (kMass) ek = exp_consts();
  for (int c = c0; c < c1; ++c) {
    float vals[kPer];
    chunk_logits<kVec4>(zrow, mw, c * kChunk, v, vals, &bad);
    if (c == c0) __syncthreads();  // the cleared histogram (and tab): after the first loads are issued
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const float zq = vals[q];
      if (zq != zq) continue;  // removed, non-finite or past the row
      mx = fmaxf(mx, zq);
      const int b = (int)(order_key(zq) >> kSelShift0);
      // exp(z / tau) against 0 (the range check below discards rows where this overflows)
      if constexpr (kMass) atomicAdd(&hm[b], exp_neg_f64_tab((double)zq * tr.inv_tau, tab, ek));
      else atomicAdd(&hc[b], 1u);
    }
  }
  if (bad) atomicOr(&sb.rbad[rowg], 1u);  // rare: a row that refuses its sequence
  mx = block_max<kThreads>(mx, lds_f);
  if (tid == 0 && mx > -INFINITY) atomicMax(&sb.rkey[rowg], order_key(mx));
  uint32_t* gc = sb.cnt + rowg * kSelB0;
  double* gm = sb.mass + rowg * kSelB0;
  if (!flush_and_arrive<kMass>(hc, hm, gc, gm, &sb.arrive[rowg], (int)gridDim.y, &s_last)) return;

  // the row's last workgroup: the boundary's digit-0 bucket and the row's course
  const uint32_t rk = __hip_atomic_load(&sb.rkey[rowg], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  SelState st{};
  st.rmax = rk ? key_logit(rk) : -INFINITY;
  st.mode = kSelDone;
  st.thr = 0u;
  if (rk != 0u) {
    uint32_t cc[16];
    double w[16];
    double above, total;
    if constexpr (!kMass) {
      load_desc16<false>(gc, gm, cc, w);
      const int b = resolve_desc<kThreads, 16>(cc, w, 0.0, (double)sa.top_k, &above, &total, lds_scan, s_d, s_i);
      if (total <= (double)sa.top_k || b < 0) {
        // top-k keeps every token: top-p (if on) runs over the full row
        if (sa.top_p < 1.0) st.mode = kSelSlowPFull;
      } else {
        const uint32_t nb = __hip_atomic_load(&gc[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        st.mode = above + (double)nb <= (double)kCand ? kSelCompactK : kSelSlowK;
        st.lo = st.mode == kSelCompactK ? (uint32_t)b << kSelShift0 : (uint32_t)b;
        st.carry = above;
      }
    } else {
      const double r = (double)st.rmax * tr.inv_tau;
      st.mode = kSelSlowPFull;
      if (r >= kRef0Lo && r <= kRef0Hi) {
        load_desc16<true>(gc, gm, cc, w);
        // the bucket masses summed in a fixed order give S (against 0) for the target P·S
        double lsum = 0.0;
#pragma unroll
        for (int i = 0; i < 16; ++i) lsum += w[i];
        const double s0 = block_sum_f64<kThreads>(lsum, lds_scan);
        const int b = resolve_desc<kThreads, 16>(cc, w, 0.0, sa.top_p * s0, &above, &total, lds_scan, s_d, s_i);
        if (b >= 0) {
          // to the row-maximum reference: multiply by exp(-m / tau) (within fp64's range here).
          // The bucket's count is not kept: sel_finish reads it from the collected candidates.
          const double f = exp_neg_f64(-r);
          st.s1 = s0 * f;
          st.carry = above * f;
          st.lo = (uint32_t)b;
          st.mode = kSelCompactP;
        }
      }
    }
  }
  if (tid == 0) sb.state[rowg] = st;
}

// The candidate keys of kSelCompactK rows (every key from state.lo up) and kSelCompactP rows
// (the keys of digit-0 bucket state.lo); other rows' workgroups return at once. One chunk per
// workgroup and one slot reservation per workgroup (the reservations of a row serialize on its
// counter; several chunks per workgroup or one reservation per wave measured slower).
template <bool kVec4>
__global__ __launch_bounds__(kThreads) void sel_collect_kernel(const float* __restrict__ target,
                                                               const float* __restrict__ draft, int kd,
                                                               int v, Transform tr, SelBufs sb) {
  __shared__ double lds_scan[kThreads / kWave];
  __shared__ uint32_t s_base;
  const int64_t rowg = blockIdx.x;
  const int per_seq = 2 * kd + 1;
  const int64_t s = rowg / per_seq;
  const int j = (int)(rowg % per_seq);
  const int c = blockIdx.y;
  const int tid = threadIdx.x;
  const SelState st = sb.state[rowg];
  if (st.mode != kSelCompactK && st.mode != kSelCompactP) return;

  float vals[kPer];
  chunk_logits<kVec4>(row_ptr(target, draft, s, kd, j, v), mask_words(tr, s, kd, mask_row(j, kd)),
                      c * kChunk, v, vals);
  const bool from = st.mode == kSelCompactK;
  bool take[kPer];
  int mine = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const uint32_t key = order_key(vals[q]);
    take[q] = vals[q] == vals[q] && (from ? key >= st.lo : (key >> kSelShift0) == st.lo);
    mine += take[q] ? 1 : 0;
  }
  const double incl = block_inclusive_scan_f64<kThreads>((double)mine, lds_scan);
  if (tid == kThreads - 1) {
    const uint32_t tot = (uint32_t)incl;
    s_base = tot ? atomicAdd(&sb.candn[rowg], tot) : 0u;
  }
  __syncthreads();
  uint32_t slot = s_base + (uint32_t)incl - (uint32_t)mine;
  uint32_t* out = sb.cand + rowg * kCand;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    if (take[q]) {
      if (slot < (uint32_t)kCand) out[slot] = order_key(vals[q]);
      ++slot;
    }
  }
}

// ---- sel_chunk: top-k from per-chunk candidates
// The row's k-th largest key K is at least every chunk's own k-th largest (that chunk's top k
// are k keys of the row), so a chunk's keys from any lower bound L_c of its own k-th largest up
// hold every key of the chunk that the row's top-k keeps. The k-th largest of the chunk's 256
// per-thread maxima is such a bound (those k maxima are k distinct keys of the chunk), and a
// close one: the chunk's largest keys mostly sit in different threads. One workgroup per chunk
// finds it (to the top 16 bits of the key) with one wave (0 when fewer than k threads hold an allowed finite token: then every
// such token is a candidate) and writes its keys from L_c up into its own slots of the
// row's list: no histogram is shared, no counter is cleared, and the logits are read once. The
// chunk's record holds the count (kRecOver: more keys than slots, none written; kRecBad: a NaN
// or +inf in the chunk, allowed or not), L_c and the chunk's largest allowed finite key (0: none).
constexpr int kMaxSelChunks = 1024;  // records of one row fill its digit-0 count area
constexpr uint32_t kRecOver = 1u << 30, kRecBad = 1u << 31, kRecCount = kRecOver - 1u;
static_assert(4 * kMaxSelChunks <= kSelB0, "chunk records live in the digit-0 count area");

// A lower bound of the k-th largest of vals[0, kWave·kR) (LDS, kR values per lane), found by
// the calling wave alone: the largest T whose low kSearchLow bits are 0 and with at least k
// values >= T, built bit by bit from the top (each bit: kR compares whose ballots are counted
// on the scalar unit). The bits below kSearchLow (below 2^-7 of a logit's magnitude) are left
// 0: a bound a little under the k-th largest, at half the steps. Every lane returns it.
constexpr int kSearchLow = 16;
template <int kR>
__device__ __forceinline__ uint32_t wave_kth_bound(const uint32_t* vals, int k) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t x[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r) x[r] = vals[lane * kR + r];
  uint32_t t = 0u;
#pragma unroll
  for (int bit = 31; bit >= kSearchLow; --bit) {
    const uint32_t cand = t | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < kR; ++r) cnt += __popcll(__ballot(x[r] >= cand));
    if (cnt >= k) t = cand;
  }
  return t;
}

// Wave-wide max of one uint32 per lane (every lane active; every lane gets it).
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)dpp_i32<kDppQuadXor1>((int)v));
  v = max(v, (uint32_t)dpp_i32<kDppQuadXor2>((int)v));
  v = max(v, (uint32_t)dpp_i32<kDppRowRor4>((int)v));
  v = max(v, (uint32_t)dpp_i32<kDppRowRor8>((int)v));
  v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  return max(v, (uint32_t)__shfl_xor((int)v, 32));
}

template <bool kVec4>
__global__ __launch_bounds__(kThreads) void sel_chunk_kernel(const float* __restrict__ target,
                                                             const float* __restrict__ draft, int kd,
                                                             int v, Transform tr, SelBufs sb, SelArgs sa) {
  __shared__ __attribute__((aligned(16))) uint32_t tmax[kThreads];
  __shared__ double lds_scan[kThreads / kWave];
  __shared__ uint32_t s_lc, s_rk, s_bad;
  __shared__ double s_n;
  const int64_t rowg = blockIdx.x;
  const int per_seq = 2 * kd + 1;
  const int64_t s = rowg / per_seq;
  const int j = (int)(rowg % per_seq);
  const int c = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0u;
  float vals[kPer];
  int bad = 0;
  chunk_logits<kVec4>(row_ptr(target, draft, s, kd, j, v), mask_words(tr, s, kd, mask_row(j, kd)),
                      c * kChunk, v, vals, &bad);
  uint32_t key[kPer];
  uint32_t m = 0u;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    key[q] = vals[q] == vals[q] ? order_key(vals[q]) : 0u;  // 0: removed (every live key is larger)
    m = max(m, key[q]);
  }
  tmax[tid] = m;
  if (bad) s_bad = 1u;
  __syncthreads();
  if (tid < kWave) {
    // one wave: L_c (0 if fewer than k threads hold a live token) and the chunk's largest key
    const uint32_t lc = wave_kth_bound<kThreads / kWave>(tmax, sa.top_k);
    const u32x4 m4 = reinterpret_cast<const u32x4*>(tmax)[tid];
    const uint32_t rk = wave_max_u32(max(max(m4[0], m4[1]), max(m4[2], m4[3])));
    if (tid == 0) {
      s_lc = lc;
      s_rk = rk;
    }
  }
  __syncthreads();
  const uint32_t lc = s_lc;
  int mine = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) mine += (key[q] && key[q] >= lc) ? 1 : 0;
  const double incl = block_inclusive_scan_f64<kThreads>((double)mine, lds_scan);
  if (tid == kThreads - 1) s_n = incl;
  __syncthreads();
  const uint32_t n = (uint32_t)s_n;
  const bool over = n > (1u << sa.slot_log2);
  if (!over) {
    // interleaved with the other chunks' candidates, so that a contiguous run of the list holds
    // candidates of many chunks
    uint32_t* out = sb.cand + rowg * kCand + c;
    const int c2 = sa.chunk_log2;
    uint32_t slot = (uint32_t)incl - (uint32_t)mine;
#pragma unroll
    for (int q = 0; q < kPer; ++q)
      if (key[q] && key[q] >= lc) out[(size_t)(slot++) << c2] = key[q];
  }
  if (tid == 0) {
    const u32x4 rec{(over ? kRecOver : n) | (s_bad ? kRecBad : 0u), lc, s_rk, 0u};
    reinterpret_cast<u32x4*>(sb.cnt + rowg * kSelB0)[c] = rec;
  }
}

// ---- sel_finish

// Sorts keys[0, n) in LDS into descending order (bitonic network over the next power of two,
// padded with key 0, which is below every finite logit's key).
__device__ __forceinline__ void sort_desc(uint32_t* keys, int n) {
  int np = 1;
  while (np < n) np <<= 1;
  for (int i = n + (int)threadIdx.x; i < np; i += kFThreads) keys[i] = 0u;
  __syncthreads();
  for (int k = 2; k <= np; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < np; i += kFThreads) {
        const int l = i ^ j;
        if (l > i) {
          const uint32_t a = keys[i], b = keys[l];
          const bool desc = (i & k) == 0;  // this half of the merge ends descending
          if (desc ? a < b : a > b) {
            keys[i] = b;
            keys[l] = a;
          }
        }
      }
      __syncthreads();
    }
  }
}

struct FinishLds {
  double scan[kFWaves];
  double incl[kFThreads];
  double d[2];
  int i[kFWaves];
};

// top-p over the sorted candidates keys[0, lim), lim <= kSortMax: carry is the mass strictly
// above them; S is s_given, or (s_from_sum) the candidates' own total. Thread t takes the
// contiguous positions [t·per, t·per + per), so every sum runs in the sorted order. Returns the
// lowest key whose strictly-larger mass is below P·S.
__device__ __forceinline__ uint32_t topp_sorted(const uint32_t* keys, int lim, double carry, double s_given, bool s_from_sum,
                                float rmax, double inv_tau, double p, FinishLds& L) {
  constexpr int kMaxPer = (kSortMax + kFThreads - 1) / kFThreads;
  const int tid = threadIdx.x;
  const int per = (lim + kFThreads - 1) / kFThreads;
  const int i0 = tid * per;
  double e[kMaxPer];
  double local = 0.0;
#pragma unroll
  for (int q = 0; q < kMaxPer; ++q) {
    const int i = i0 + q;
    e[q] = (q < per && i < lim) ? exp_neg_f64(((double)key_logit(keys[i]) - (double)rmax) * inv_tau) : 0.0;
    local += e[q];
  }
  const double incl = block_inclusive_scan_f64<kFThreads>(local, L.scan);
  L.incl[tid] = incl;
  __syncthreads();
  const double s = s_from_sum ? L.incl[kFThreads - 1] : s_given;
  const double tgt = p * s;
  double run = carry + (tid > 0 ? L.incl[tid - 1] : 0.0);
  int best = -1;
#pragma unroll
  for (int q = 0; q < kMaxPer; ++q) {
    const int i = i0 + q;
    if (q < per && i < lim) {
      const bool start = i == 0 || keys[i - 1] != keys[i];
      if (start && run < tgt) best = i;
      run += e[q];
    }
  }
  best = block_max_i32<kFThreads>(best, L.i);
  return keys[best >= 0 ? best : 0];
}

// The tokens a finishing pass walks: the row itself (global memory, with its mask) or the
// collected candidate keys in LDS. each(f) calls f(z, key) for every allowed finite token.
template <bool kVec4>
struct RowSrc {
  const float* z;
  const uint32_t* mw;
  int v;
  template <class F>
  __device__ void each(F&& f) const {
    auto one = [&](float zz, bool allowed) {
      if (allowed && zz > -INFINITY && zz < INFINITY) f(zz, order_key(zz));
    };
    if constexpr (kVec4) {
      for (int e4 = 4 * (int)threadIdx.x; e4 < v; e4 += 4 * kFThreads) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(z + e4);
        const uint32_t w = mw ? mw[e4 >> 5] : 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < 4; ++i) one(t[i], ((w >> ((e4 + i) & 31)) & 1u) != 0u);
      }
    } else {
      for (int t = threadIdx.x; t < v; t += kFThreads)
        one(z[t], mw ? ((mw[t >> 5] >> (t & 31)) & 1u) != 0u : true);
    }
  }
};

struct KeySrc {
  const uint32_t* keys;
  int n;
  template <class F>
  __device__ void each(F&& f) const {
    for (int i = threadIdx.x; i < n; i += kFThreads) {
      const uint32_t key = keys[i];
      f(key_logit(key), key);
    }
  }
};

// One radix pass of the finishing workgroup: histogram of the digit (key >> shift) & (nb - 1)
// of the source's tokens whose key is at least keep_lo and, when mshift < 32, whose
// key >> mshift equals mval; counts, and with kMass masses exp((z - rmax) / tau). Returns the
// masses' total over the selected tokens (0 without kMass).
template <bool kMass, class Src>
__device__ __forceinline__ double fin_hist(const Src& src, uint32_t keep_lo, int mshift, uint32_t mval, int shift, int nb,
                           float rmax, double inv_tau, uint32_t* hc, double* hm, FinishLds& L) {
  for (int b = threadIdx.x; b < nb; b += kFThreads) {
    hc[b] = 0u;
    if constexpr (kMass) hm[b] = 0.0;
  }
  __syncthreads();
  double acc = 0.0;
  src.each([&](float zz, uint32_t key) {
    if (key < keep_lo || (mshift < 32 && (key >> mshift) != mval)) return;
    const int b = (int)((key >> shift) & (uint32_t)(nb - 1));
    atomicAdd(&hc[b], 1u);
    if constexpr (kMass) {
      const double e = exp_neg_f64(((double)zz - (double)rmax) * inv_tau);
      atomicAdd(&hm[b], e);
      acc += e;
    }
  });
  double tot = 0.0;
  if constexpr (kMass) tot = block_sum_f64<kFThreads>(acc, L.scan);
  __syncthreads();
  return tot;
}

// The boundary bucket of an LDS histogram of nb buckets (1024 or 4096) walked downwards.
template <bool kMass>
__device__ __forceinline__ int fin_resolve(const uint32_t* hc, const double* hm, int nb, double carry, double target,
                           double* above, FinishLds& L) {
  double total;
  if (nb == kSelB0) {
    constexpr int kP = kSelB0 / kFThreads;
    uint32_t c[kP];
    double w[kP];
#pragma unroll
    for (int i = 0; i < kP; ++i) {
      const int b = nb - 1 - ((int)threadIdx.x * kP + i);
      c[i] = hc[b];
      w[i] = kMass ? hm[b] : (double)c[i];
    }
    return resolve_desc<kFThreads, kP>(c, w, carry, target, above, &total, L.scan, L.d, L.i);
  }
  constexpr int kP = (1 << kSelBits1) / kFThreads;
  uint32_t c[kP];
  double w[kP];
#pragma unroll
  for (int i = 0; i < kP; ++i) {
    const int b = nb - 1 - ((int)threadIdx.x * kP + i);
    c[i] = hc[b];
    w[i] = kMass ? hm[b] : (double)c[i];
  }
  return resolve_desc<kFThreads, kP>(c, w, carry, target, above, &total, L.scan, L.d, L.i);
}

// Digits 1 and 2 of a walk whose digit-0 bucket (prefix) and carry are known; returns the
// threshold key. A bucket that does not resolve (only if the row changed during the call)
// keeps every token of the prefix.
template <bool kMass, class Src>
__device__ __forceinline__ uint32_t fin_digits12(const Src& src, uint32_t keep_lo, uint32_t prefix, double carry, double target,
                                 float rmax, double inv_tau, uint32_t* hc, double* hm, FinishLds& L) {
  for (int d = 1; d <= 2; ++d) {
    const int mshift = d == 1 ? kSelShift0 : kSelBits1;
    const int shift = d == 1 ? kSelBits1 : 0;
    fin_hist<kMass>(src, keep_lo, mshift, prefix, shift, 1 << kSelBits1, rmax, inv_tau, hc, hm, L);
    double above = carry;
    const int b = fin_resolve<kMass>(hc, hm, 1 << kSelBits1, carry, target, &above, L);
    prefix = (prefix << kSelBits1) | (uint32_t)(b >= 0 ? b : 0);
    carry = above;
  }
  return prefix;
}

// top-p over the source's tokens with key >= keep_lo (the tokens top-k kept), all three digits.
template <class Src>
__device__ __forceinline__ uint32_t fin_topp(const Src& src, uint32_t keep_lo, double p, float rmax, double inv_tau, uint32_t* hc,
                             double* hm, FinishLds& L) {
  const double s1 = fin_hist<true>(src, keep_lo, 32, 0u, kSelShift0, kSelB0, rmax, inv_tau, hc, hm, L);
  double above = 0.0;
  const int b = fin_resolve<true>(hc, hm, kSelB0, 0.0, p * s1, &above, L);
  if (b < 0) return keep_lo;
  return fin_digits12<true>(src, keep_lo, (uint32_t)b, above, p * s1, rmax, inv_tau, hc, hm, L);
}

// top-k over the source's tokens with key >= keep_lo, all three digits (keep_lo when there are
// none).
template <class Src>
__device__ __forceinline__ uint32_t fin_select_k(const Src& src, uint32_t keep_lo, double k, float rmax, double inv_tau,
                                                 uint32_t* hc, double* hm, FinishLds& L) {
  fin_hist<false>(src, keep_lo, 32, 0u, kSelShift0, kSelB0, rmax, inv_tau, hc, hm, L);
  double above = 0.0;
  const int b = fin_resolve<false>(hc, hm, kSelB0, 0.0, k, &above, L);
  if (b < 0) return keep_lo;
  return fin_digits12<false>(src, keep_lo, (uint32_t)b, above, k, rmax, inv_tau, hc, hm, L);
}

// Block-wide max of one uint32 per thread (kT threads); lds: kT / kWave ints.
template <int kT>
__device__ inline uint32_t block_max_u32(uint32_t v, int* lds) {
  return (uint32_t)block_max_i32<kT>((int)(v ^ 0x80000000u), lds) ^ 0x80000000u;
}

// Moves the keys of keys[0, n) that are at least lo to the front, in their order; returns
// their number. Thread t takes the contiguous positions [t·per, t·per + per).
__device__ __forceinline__ int compact_keys(uint32_t* keys, int n, uint32_t lo, FinishLds& L) {
  constexpr int kMax = kCand / kFThreads;
  const int per = (n + kFThreads - 1) / kFThreads;
  const int i0 = (int)threadIdx.x * per;
  uint32_t r[kMax];
  int mine = 0;
#pragma unroll
  for (int q = 0; q < kMax; ++q) {
    const int i = i0 + q;
    r[q] = (q < per && i < n) ? keys[i] : 0u;
    mine += (q < per && i < n && r[q] >= lo) ? 1 : 0;
  }
  // the scan's barriers order every read above before the writes below
  const double incl = block_inclusive_scan_f64<kFThreads>((double)mine, L.scan);
  int o = (int)incl - mine;
#pragma unroll
  for (int q = 0; q < kMax; ++q)
    if (q < per && i0 + q < n && r[q] >= lo) keys[o++] = r[q];
  if (threadIdx.x == kFThreads - 1) L.i[0] = (int)incl;
  __syncthreads();
  const int m = L.i[0];
  __syncthreads();
  return m;
}

// A lower bound of the k-th largest of keys[0, n) (k <= kFThreads): the k-th largest of the
// threads' maxima over contiguous runs of the keys (those k maxima are k distinct keys), to its
// top 16 bits; 0 when fewer than k threads hold a key. tm: kFThreads words of LDS, 16-byte aligned.
__device__ __forceinline__ uint32_t maxima_bound(const uint32_t* keys, int n, int k, uint32_t* tm, FinishLds& L) {
  const int tid = threadIdx.x;
  const int per = (n + kFThreads - 1) / kFThreads;
  uint32_t m = 0u;
  for (int i = tid * per; i < min(n, tid * per + per); ++i) m = max(m, keys[i]);
  tm[tid] = m;
  __syncthreads();
  if (tid < kWave) {
    const uint32_t b = wave_kth_bound<kFThreads / kWave>(tm, k);
    if (tid == 0) L.i[0] = (int)b;
  }
  __syncthreads();
  const uint32_t b = (uint32_t)L.i[0];
  __syncthreads();
  return b;
}

// sel_chunk's candidates of one row, cut to the keys from a lower bound of the row's k-th
// largest up, into keys[0, n) (in no particular order). The bound is the larger of L* = max L_c
// (every L_c is at most the row's k-th largest key) and the k-th largest of the threads' maxima
// over the candidates from L* up, to its top 16 bits (those k maxima are k distinct candidates,
// and the candidates hold every key the row's top-k keeps). Returns n, or -1 when a chunk had
// more candidates than its slots. *rk: the row's largest allowed finite key (0: none); *bad: a
// NaN or +inf in the row. LDS: cnt_l (kMaxSelChunks words), tm (kFThreads words, 16-byte
// aligned), red (4·kFWaves + 1 words). The records and the slots load together.
__device__ __forceinline__ int gather_chunks(const SelBufs& sb, int64_t rowg, int chunks, int slot_log2, int c2, int k,
                                             uint32_t* keys, uint32_t* cnt_l, uint32_t* tm, uint32_t* red,
                                             uint32_t* rk, bool* bad) {
  constexpr int kRecPer = kMaxSelChunks / kFThreads;
  constexpr int kVecPer = kCand / 4 / kFThreads;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const u32x4* rec = reinterpret_cast<const u32x4*>(sb.cnt + rowg * kSelB0);
  const u32x4* cs = reinterpret_cast<const u32x4*>(sb.cand + rowg * kCand);
  const int slots = 1 << (slot_log2 + c2);  // list position i·2^c2 + c: candidate i of chunk c
  u32x4 r[kRecPer], kv[kVecPer];
#pragma unroll
  for (int i = 0; i < kRecPer; ++i) {
    const int c = tid + kFThreads * i;
    r[i] = c < chunks ? rec[c] : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < kVecPer; ++u) {
    const int e4 = tid + kFThreads * u;
    kv[u] = 4 * e4 < slots ? cs[e4] : u32x4{0u, 0u, 0u, 0u};
  }
  int flags = 0;
  uint32_t lmax = 0u, kmax = 0u;
#pragma unroll
  for (int i = 0; i < kRecPer; ++i) {
    const int c = tid + kFThreads * i;
    if (c < chunks) {
      cnt_l[c] = r[i][0] & kRecCount;
      flags |= (int)(r[i][0] >> 30);
      lmax = max(lmax, r[i][1]);
      kmax = max(kmax, r[i][2]);
    }
  }
  flags = wave_or(flags);
  lmax = wave_max_u32(lmax);
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    red[wave] = (uint32_t)flags;
    red[kFWaves + wave] = lmax;
    red[2 * kFWaves + wave] = kmax;
  }
  __syncthreads();  // the chunk counts and the waves' partials
  uint32_t f = 0u, lstar = 0u, kx = 0u;
#pragma unroll
  for (int w = 0; w < kFWaves; ++w) {
    f |= red[w];
    lstar = max(lstar, red[kFWaves + w]);
    kx = max(kx, red[2 * kFWaves + w]);
  }
  *rk = kx;
  *bad = (f & (kRecBad >> 30)) != 0u;
  if (f & (kRecOver >> 30)) return -1;
  // this thread's candidates from L* up and their maximum
  const int cmask = (1 << c2) - 1;
  uint32_t take = 0u;  // bit 4u + i: kv[u][i]
  uint32_t m = 0u;
#pragma unroll
  for (int u = 0; u < kVecPer; ++u) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * (tid + kFThreads * u) + i;
      const int c = e & cmask;
      const bool ok = e < slots && c < chunks && (uint32_t)(e >> c2) < cnt_l[c] && kv[u][i] >= lstar;
      take |= ok ? 1u << (4 * u + i) : 0u;
      m = ok ? max(m, kv[u][i]) : m;
    }
  }
  tm[tid] = m;
  __syncthreads();
  if (wave == 0) {
    const uint32_t b = wave_kth_bound<kFThreads / kWave>(tm, k);
    if (lane == 0) red[3 * kFWaves] = b;
  }
  __syncthreads();
  const uint32_t lo = max(lstar, red[3 * kFWaves]);
  int mine = 0;
#pragma unroll
  for (int u = 0; u < kVecPer; ++u) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t bit = 1u << (4 * u + i);
      if ((take & bit) && kv[u][i] < lo) take &= ~bit;
      mine += (take & bit) ? 1 : 0;
    }
  }
  // positions: a scan inside each wave, then the wave totals (one barrier)
  const int incl = (int)wave_inclusive_scan_f64((double)mine);
  if (lane == kWave - 1) red[3 * kFWaves + 1 + wave] = (uint32_t)incl;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kFWaves; ++w) {
    const int t = (int)red[3 * kFWaves + 1 + w];
    base += w < wave ? t : 0;
    total += t;
  }
  int o = base + incl - mine;
#pragma unroll
  for (int u = 0; u < kVecPer; ++u) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (take & (1u << (4 * u + i))) keys[o++] = kv[u][i];
  }
  __syncthreads();
  return total;
}

__device__ inline double shfl_f64(double v, int src) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)b, src);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(b >> 32), src);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// The thresholds from n <= kWave candidates keys[0, n) (LDS; every key top-k keeps is among
// them) on the calling wave alone, with no barrier: a bitonic sort, one key per lane, descending;
// top-k's threshold is the k-th key (the last when n <= k); top-p (p < 1) then takes the lowest
// key whose strictly-larger mass is below P·S among the keys top-k kept (masses
// exp((z - rmax) / tau), S their sum, both summed in the sorted order by a wave scan). With
// with_stats, the row's statistics as write_row_stats writes them. Returns the threshold (every lane).
__device__ __forceinline__ uint32_t wave_tail(const uint32_t* keys, int n, int k, double p, float rmax, double inv_tau,
                                              const double* tab, const SelStats& ss, bool with_stats, int64_t rowg,
                                              const DraftLogit& dl) {
  if (n <= 0) return 0u;
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t x = lane < n ? keys[lane] : 0u;  // 0 is below every live key: the padding sorts last
#pragma unroll
  for (int kk = 2; kk <= kWave; kk <<= 1) {
#pragma unroll
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      const uint32_t y = (uint32_t)__shfl_xor((int)x, jj);
      const bool lower = (lane & jj) == 0;  // this lane holds the pair's lower position
      const bool desc = (lane & kk) == 0;   // this block of kk ends descending
      x = lower == desc ? max(x, y) : min(x, y);
    }
  }
  const uint32_t thr_k = (uint32_t)__shfl((int)x, min(k, n) - 1);
  uint32_t thr = thr_k;
  const bool kept_k = lane < n && x >= thr_k;
  const double e = kept_k ? exp_neg_f64_tab(((double)key_logit(x) - (double)rmax) * inv_tau, tab) : 0.0;
  if (p < 1.0) {
    const double incl = wave_inclusive_scan_f64(e);
    const double tgt = p * readlane_f64(incl, kWave - 1);
    const double run = shfl_f64(incl, lane > 0 ? lane - 1 : 0);
    const uint32_t xp = (uint32_t)__shfl((int)x, lane > 0 ? lane - 1 : 0);
    const bool start = kept_k && (lane == 0 || xp != x);
    const uint64_t q = __ballot(start && (lane == 0 ? 0.0 : run) < tgt);
    thr = (uint32_t)__shfl((int)x, q ? 63 - __clzll(q) : 0);
  }
  if (with_stats) {
    const double sum = readlane_f64(wave_sum_f64(lane < n && x >= thr ? e : 0.0), 0);
    for (int c = lane; c < ss.chunks; c += kWave) {
      const size_t o = (size_t)rowg * ss.chunks + c;
      ss.cmax[o] = c == 0 ? rmax : -INFINITY;
      ss.csum[o] = c == 0 ? sum : 0.0;
      ss.cbad[o] = 0;
    }
    if (lane == 0) dl.put(ss, rowg, thr);
  }
  return thr;
}

// The stats kernel's outputs for a row whose kept set is known here, none of the row's logits
// NaN or +inf: the row maximum and S = sum exp((z - max) / tau) over the kept set in chunk 0 and
// empty other chunks, which the decide kernel combines to the same (max, S); the live logit of
// the row's draft token (threshold thr). Every thread calls it with the same sum.
__device__ __forceinline__ void put_row_stats(double sum, uint32_t thr, float rmax, const SelStats& ss, int64_t rowg,
                                              const DraftLogit& dl) {
  const int tid = threadIdx.x;
  for (int c = tid; c < ss.chunks; c += kFThreads) {
    const size_t o = (size_t)rowg * ss.chunks + c;
    ss.cmax[o] = c == 0 ? rmax : -INFINITY;
    ss.csum[o] = c == 0 ? sum : 0.0;
    ss.cbad[o] = 0;
  }
  if (tid == 0) dl.put(ss, rowg, thr);
}

// put_row_stats for a kept set of carry (the mass of the kept tokens outside the list) plus the
// keys of keys[0, n) from thr up, summed by a fixed-order block sum over the list's order (one
// key per thread for n <= kFThreads, so a sorted list gives a sum in the sorted order).
__device__ __forceinline__ void write_row_stats(const uint32_t* keys, int n, uint32_t thr, double carry, float rmax,
                                                double inv_tau, const double* tab, const SelStats& ss,
                                                int64_t rowg, const DraftLogit& dl, FinishLds& L) {
  double e = 0.0;
  for (int i = threadIdx.x; i < n; i += kFThreads)
    if (keys[i] >= thr) e += exp_neg_f64_tab(((double)key_logit(keys[i]) - (double)rmax) * inv_tau, tab);
  const double sum = carry + block_sum_f64<kFThreads>(e, L.scan);
  put_row_stats(sum, thr, rmax, ss, rowg, dl);
}

template <bool kVec4>
__global__ __launch_bounds__(kFThreads) void sel_finish_kernel(const float* __restrict__ target,
                                                               const float* __restrict__ draft, int kd,
                                                               int v, Transform tr, SelBufs sb,
                                                               SelArgs sa, SelStats ss) {
  __shared__ uint32_t keys[kCand];  // the candidates
  __shared__ __attribute__((aligned(16))) uint32_t hc[kSelB0];  // radix passes: counts (also the
                                                                 // chunk counts, the thread maxima)
  __shared__ double hm[kSelB0];     // radix passes: masses
  __shared__ FinishLds L;
  __shared__ double tab[32];        // 2^(j/32) for the row statistics: written by wave 0, which the
                                    // one-wave tail runs on; the other waves read it after a barrier
  __shared__ uint32_t red[4 * kFWaves + 1];
  const int64_t rowg = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < 32) tab[tid] = kExp2Table32[tid];
  const int per_seq = 2 * kd + 1;
  const int64_t s = rowg / per_seq;
  const int j = (int)(rowg % per_seq);
  const bool use_p = sa.top_p < 1.0;
  const double kf = (double)sa.top_k;
  DraftLogit dl;
  if (tid == 0) dl.load_token(ss, s, j, kd, v);  // first: its wait is absorbed by the next one
  bool stats_done = false;
  uint32_t thr = 0u;
  SelState st{};
  bool bad_row;
  int n = 0;             // candidates in keys[0, n) (compact modes)
  bool digit0 = false;   // kSelCompactK: the boundary's digit-0 bucket (st.lo) and carry are known
  if (sa.slot_log2 > 0) {
    uint32_t rk;
    n = gather_chunks(sb, rowg, sa.chunks, sa.slot_log2, sa.chunk_log2, sa.top_k, keys, hc, hc + kMaxSelChunks, red,
                      &rk, &bad_row);
    st.rmax = rk ? key_logit(rk) : -INFINITY;
    st.mode = rk == 0u ? kSelDone : (n < 0 ? kSelSlowKFull : kSelCompactK);
  } else {
    st = sb.state[rowg];
    bad_row = sb.rbad[rowg] != 0u;
    if (st.mode == kSelCompactK || st.mode == kSelCompactP) {
      n = (int)sb.candn[rowg];
      if (n > kCand) {
        // more candidates than the list holds (top-p buckets are not counted ahead): radix
        // passes over the row
        if (st.mode == kSelCompactK) {
          st.mode = kSelSlowK;
          st.lo >>= kSelShift0;
        } else {
          st.mode = kSelSlowP;
        }
      } else {
        const uint32_t* src = sb.cand + rowg * kCand;
        for (int i = tid; i < n; i += kFThreads) keys[i] = src[i];
        __syncthreads();
        digit0 = st.mode == kSelCompactK;
      }
    }
  }
  if (tid == 0) dl.load_logit(row_ptr(target, draft, s, kd, j, v), mask_words(tr, s, kd, mask_row(j, kd)));
  if (st.mode == kSelCompactK) {
    // keys[0, n) hold every key the row's top-k keeps; cut them towards the kept set
    uint32_t thr_k = 0u;
    if (n > kSortMax && sa.top_k <= kFThreads) n = compact_keys(keys, n, maxima_bound(keys, n, sa.top_k, hc, L), L);
    if (n > kSortMax) {
      const KeySrc ks{keys, n};
      thr_k = digit0 ? fin_digits12<false>(ks, 0u, st.lo >> kSelShift0, st.carry, kf, st.rmax, tr.inv_tau, hc, hm, L)
                     : fin_select_k(ks, 0u, kf, st.rmax, tr.inv_tau, hc, hm, L);
      n = compact_keys(keys, n, thr_k, L);  // now exactly the kept set
      if (n > kSortMax) {
        thr = use_p ? fin_topp(KeySrc{keys, n}, thr_k, sa.top_p, st.rmax, tr.inv_tau, hc, hm, L) : thr_k;
        n = -1;  // done, without the row's statistics
      }
    }
    const bool with_stats = ss.cmax && n > 0 && !bad_row;
    if (n >= 0 && n <= kWave) {
      // the usual case: one wave, no barrier
      if (tid < kWave)
        thr = wave_tail(keys, n, sa.top_k, use_p ? sa.top_p : 1.0, st.rmax, tr.inv_tau, tab,
                        ss, with_stats, rowg, dl);
      stats_done = with_stats;
    } else if (n > kWave) {
      sort_desc(keys, n);
      // the candidates hold the row's n largest keys that top-k can keep: its threshold is the k-th
      thr_k = keys[min(sa.top_k, n) - 1];
      thr = thr_k;
      if (use_p) {
        // top-p on the tokens top-k kept: the first m sorted keys
        int last = -1;
        for (int i = tid; i < n; i += kFThreads)
          if (keys[i] >= thr_k && (i + 1 == n || keys[i + 1] < thr_k)) last = i;
        const int m = block_max_i32<kFThreads>(last, L.i) + 1;
        thr = topp_sorted(keys, m, 0.0, 0.0, true, st.rmax, tr.inv_tau, sa.top_p, L);
      }
      // the kept set is here, sorted: the row's statistics too (the stats kernel skips it)
      if (with_stats) {
        write_row_stats(keys, n, thr, 0.0, st.rmax, tr.inv_tau, tab, ss, rowg, dl, L);
        stats_done = true;
      }
    }
  } else if (st.mode == kSelCompactP) {
    if (n <= kSortMax) {
      sort_desc(keys, n);
      if (n > 0) thr = topp_sorted(keys, n, st.carry, st.s1, false, st.rmax, tr.inv_tau, sa.top_p, L);
    } else {
      const KeySrc ks{keys, n};
      thr = fin_digits12<true>(ks, 0u, st.lo, st.carry, sa.top_p * st.s1, st.rmax, tr.inv_tau, hc, hm, L);
    }
    // the kept set: every token above the boundary bucket (mass st.carry) and the bucket's keys
    // from thr up, so the row's statistics are known here too (the stats kernel skips the row)
    if (ss.cmax && n > 0 && !bad_row) {
      write_row_stats(keys, n, thr, st.carry, st.rmax, tr.inv_tau, tab, ss, rowg, dl, L);
      stats_done = true;
    }
  } else if (st.mode != kSelDone) {
    const RowSrc<kVec4> rs{row_ptr(target, draft, s, kd, j, v), mask_words(tr, s, kd, mask_row(j, kd)), v};
    if (st.mode == kSelSlowP) {
      thr = fin_digits12<true>(rs, 0u, st.lo, st.carry, sa.top_p * st.s1, st.rmax, tr.inv_tau, hc, hm, L);
    } else {
      if (st.mode == kSelSlowK)
        thr = fin_digits12<false>(rs, 0u, st.lo, st.carry, kf, st.rmax, tr.inv_tau, hc, hm, L);
      else if (st.mode == kSelSlowKFull)
        thr = fin_select_k(rs, 0u, kf, st.rmax, tr.inv_tau, hc, hm, L);
      if (use_p) thr = fin_topp(rs, thr, sa.top_p, st.rmax, tr.inv_tau, hc, hm, L);
    }
  } else {
    thr = st.thr;  // kSelDone
  }
  if (tid == 0) {
    sb.thr[rowg] = thr;
    if (ss.sdone) ss.sdone[rowg] = stats_done ? 1u : 0u;
  }
}

// ---------------------------------------------------------------- decide + piece totals
// kPrefetch: small calls fetch every candidate final row with the statistics (one
// workgroup per CU holds the extra registers); large calls load only the rows the
// draw needs and fit two workgroups per CU. Large calls also give a workgroup kPer
// consecutive pieces (one decision, then the pieces' row loads together), so the
// statistics combine is not repeated per piece and the grid is about one resident round.
template <bool kPrefetch, bool kT, int kPer = kPrefetch ? 1 : 4>
__global__ __launch_bounds__(kWThreads, kPrefetch ? 4 : 8) void decide_kernel(
    const float* __restrict__ target, const float* __restrict__ draft,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms, int kd, int v,
    int chunks, int pieces, Workspace ws, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_num, int32_t* __restrict__ flags, int vec4, Transform tr) {
  __shared__ double smax[kMaxRows];
  __shared__ double ssum[kMaxRows];
  __shared__ int sbad[kMaxRows];
  __shared__ double lds_d[2 * kWThreads / kWave];
  __shared__ int s_n;
  __shared__ double tab[32];  // visible after the barrier before the piece totals
  if (threadIdx.x < 32) tab[threadIdx.x] = kExp2Table32[threadIdx.x];
  const int c = blockIdx.x;
  const int64_t s = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int per_seq = 2 * kd + 1;

  // For small batches with K <= 4, every candidate final row's 4 logits of this
  // thread are fetched now, together with the statistics, so step 3 needs no
  // further memory trip. That reads all 2K+1 rows again, so large batches (where
  // bandwidth, not latency, bounds the call) load only the rows step 3 needs.
  constexpr int kPre = kPrefetch ? 9 : 1;
  const int t0w = c * kPer * kPiece + threadIdx.x * kWPer;  // (prefetch: kPer = 1)
  const bool pre = kPrefetch && vec4 && kd <= 4 && t0w + kWPer <= v;
  f32x4 prow[kPre];
#pragma unroll
  for (int r = 0; r < kPre; ++r) {
    prow[r] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (pre && r < per_seq) prow[r] = *reinterpret_cast<const f32x4*>(row_ptr(target, draft, s, kd, r, v) + t0w);
  }

  // inputs of the decisions, loaded together with the chunk statistics below
  int32_t x = -1;
  float ui = 0.f, gzt = 0.f, gzd = 0.f;
  if (wave == 0 && lane < kd) {
    x = tokens[(size_t)s * kd + lane];
    ui = uniforms[(size_t)s * (kd + 1) + lane];
    gzt = ws.gz[(size_t)s * per_seq + lane];
    gzd = ws.gz[(size_t)s * per_seq + kd + 1 + lane];
  }

  // 1. per-row max and sum over the chunk statistics. With seg = chunks rounded up
  //    to a power of two (<= 64), in pass r thread t loads chunk t % seg of row
  //    r * (kWThreads / seg) + t / seg, and each row is reduced by xor-shuffles
  //    inside its segment; the loads of up to kPassBatch passes are issued together.
  int seg = 1;
  while (seg < chunks) seg <<= 1;
  if (kPrefetch && chunks <= 4 * kQuadChunks && per_seq <= kWThreads / 4) {
    // small calls: four threads per row; thread qd of row j folds chunks qd, qd + 4, ... in
    // registers (all loads issued together), and the quad is combined by two DPP exchanges
    const int j = (int)threadIdx.x >> 2, qd = (int)threadIdx.x & 3;
    const bool rowok = j < per_seq;
    const size_t o = ((size_t)s * per_seq + (rowok ? j : 0)) * chunks;
    float cm[kQuadChunks];
    double cs[kQuadChunks];
    int cb[kQuadChunks];
#pragma unroll
    for (int i = 0; i < kQuadChunks; ++i) {
      const int cc = qd + 4 * i;
      const bool live = rowok && cc < chunks;
      const size_t oo = o + (live ? cc : 0);
      cm[i] = ws.cmax[oo];
      cs[i] = ws.csum[oo];
      cb[i] = ws.cbad[oo];
      cm[i] = live ? cm[i] : -INFINITY;
      cs[i] = live ? cs[i] : 0.0;
      cb[i] = live ? cb[i] : 0;
    }
    float m = -INFINITY;
    int bad = 0;
#pragma unroll
    for (int i = 0; i < kQuadChunks; ++i) {
      m = fmaxf(m, cm[i]);
      bad |= cb[i];
    }
    m = fmaxf(m, dpp_f32<kDppQuadXor1>(m));
    m = fmaxf(m, dpp_f32<kDppQuadXor2>(m));
    bad |= dpp_i32<kDppQuadXor1>(bad);
    bad |= dpp_i32<kDppQuadXor2>(bad);
    bad |= (m == -INFINITY);
    double sum = 0.0;
#pragma unroll
    for (int i = 0; i < kQuadChunks; ++i) {
      const double dm = kT ? ((double)cm[i] - (double)m) * tr.inv_tau : (double)cm[i] - (double)m;
      sum += (!bad && cs[i] > 0.0) ? cs[i] * exp_neg_f64(dm) : 0.0;
    }
    sum += dpp_f64<kDppQuadXor1>(sum);  // the same total on every thread of the quad
    sum += dpp_f64<kDppQuadXor2>(sum);
    if (rowok && qd == 0) {
      smax[j] = (double)m;
      ssum[j] = sum;
      sbad[j] = bad;
    }
  } else if (seg <= kWave) {
    const int rpp = kWThreads / seg;  // rows per pass
    const int passes = (per_seq + rpp - 1) / rpp;
    const int cc = threadIdx.x % seg;
    for (int p0 = 0; p0 < passes; p0 += kPassBatch) {
      float cm[kPassBatch];
      double cs[kPassBatch];
      int cb[kPassBatch];
#pragma unroll
      for (int r = 0; r < kPassBatch; ++r) {
        const int j = (p0 + r) * rpp + (int)threadIdx.x / seg;
        const bool live = j < per_seq && cc < chunks;
        const size_t o = ((size_t)s * per_seq + (live ? j : 0)) * chunks + (live ? cc : 0);
        cm[r] = live ? ws.cmax[o] : -INFINITY;
        cs[r] = live ? ws.csum[o] : 0.0;
        cb[r] = live ? ws.cbad[o] : 0;
      }
#pragma unroll
      for (int r = 0; r < kPassBatch; ++r) {
        const int j = (p0 + r) * rpp + (int)threadIdx.x / seg;
        float m = cm[r];
        int bad = cb[r];
        for (int off = 1; off < seg; off <<= 1) {
          m = fmaxf(m, __shfl_xor(m, off));
          bad |= __shfl_xor(bad, off);
        }
        bad |= (m == -INFINITY);
        const double dm = kT ? ((double)cm[r] - (double)m) * tr.inv_tau : (double)cm[r] - (double)m;
        double sum = (!bad && cs[r] > 0.0) ? cs[r] * exp_neg_f64(dm) : 0.0;
        for (int off = 1; off < seg; off <<= 1) sum += __shfl_xor(sum, off);
        if (j < per_seq && cc == 0) {
          smax[j] = (double)m;
          ssum[j] = sum;
          sbad[j] = bad;
        }
      }
    }
  } else {
    for (int j = wave; j < per_seq; j += kWThreads / kWave) {
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
          const double dm = kT ? ((double)ws.cmax[o + cc] - m64) * tr.inv_tau
                               : (double)ws.cmax[o + cc] - m64;
          if (cs > 0.0) sum += cs * exp_neg_f64(dm);
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
  }
  __syncthreads();

  // 2. decisions: lane i of wave 0 tests draft position i; n = first rejection
  if (wave == 0) {
    int bad = 0;
    for (int j = lane; j < per_seq; j += kWave) bad |= sbad[j];
    bad = __any(bad);
    int f = 0;
    bool acc = true;
    if (!bad && lane < kd) {
      double a = 0.0;
      if (x < 0 || x >= v) {
        f |= MXS_FLAG_TOKEN_RANGE;
      } else {
        // the draft token's logits were gathered by the stats kernel (-inf if removed)
        const double itau = kT ? tr.inv_tau : 1.0;
        const double q = exp_neg_f64(((double)gzd - smax[kd + 1 + lane]) * itau) / ssum[kd + 1 + lane];
        const double p = exp_neg_f64(((double)gzt - smax[lane]) * itau) / ssum[lane];
        if (q == 0.0) {
          f |= MXS_FLAG_Q_ZERO;
        } else {
          a = p / q;
          a = a < 1.0 ? a : 1.0;
        }
      }
      acc = (double)ui < a;
    }
    const unsigned long long rej = __ballot(!acc);  // lanes >= kd vote "accept"
    const int n = bad ? -1 : (rej ? __ffsll(rej) - 1 : kd);
    if (lane > n) f = 0;  // positions after the first rejection are not examined
    f = (__ballot(f & MXS_FLAG_TOKEN_RANGE) ? MXS_FLAG_TOKEN_RANGE : 0) |
        (__ballot(f & MXS_FLAG_Q_ZERO) ? MXS_FLAG_Q_ZERO : 0);
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

  // 3. piece total of the final weights: thread totals in token order, then
  // the same block scan the sample kernel uses, so both see identical totals
  const int n = s_n;
  // the final rows' laws, the same for every piece of this workgroup (set up once)
  FinalRows fr;
  fr.tab = tab;
  fr.ek = exp_consts();
  if (n >= 0) {
    fr.zt = row_ptr(target, draft, s, kd, n, v);
    fr.zd = n < kd ? row_ptr(target, draft, s, kd, kd + 1 + n, v) : nullptr;
    fr.mt = smax[n];
    fr.inv_st = 1.0 / ssum[n];
    fr.md = n < kd ? smax[kd + 1 + n] : 0.0;
    fr.inv_sd = n < kd ? 1.0 / ssum[kd + 1 + n] : 0.0;
    if constexpr (kT) {
      fr.inv_tau = tr.inv_tau;
      fr.thr_t = tr.thr ? tr.thr[(size_t)s * per_seq + n] : 0u;
      fr.thr_d = (tr.thr && n < kd) ? tr.thr[(size_t)s * per_seq + kd + 1 + n] : 0u;
      fr.mw = mask_words(tr, s, kd, n);
    }
  }
#pragma unroll
  for (int pc = 0; pc < kPer; ++pc) {
    const int cp = c * kPer + pc;  // this piece (uniform: the loop holds block scans)
    if (cp >= pieces) break;
    const int t0p = cp * kPiece + threadIdx.x * kWPer;
    double a = 0.0, b = 0.0;
    if (n >= 0) {
      double wf[kWPer], wp[kWPer];
      if (pre) {
        float zt[kWPer], zd[kWPer];
        f32x4 at = prow[0], ad = prow[0];
  #pragma unroll
        for (int r = 0; r < kPre; ++r) {  // select without indexing registers dynamically
          if (r == n) at = prow[r];
          if (r == kd + 1 + n) ad = prow[r];
        }
  #pragma unroll
        for (int j = 0; j < kWPer; ++j) {
          zt[j] = at[j];
          zd[j] = ad[j];
          if constexpr (kT) {
            zt[j] = live_logit(zt[j], t0w + j, fr.mw, fr.thr_t);
            zd[j] = live_logit(zd[j], t0w + j, fr.mw, fr.thr_d);
          }
        }
        weights_from<kT>(fr, zt, zd, wf, wp);
      } else {
        thread_weights<kT>(fr, t0p, v, vec4, wf, wp);
      }
  #pragma unroll
      for (int j = 0; j < kWPer; ++j) {
        a += wf[j];
        b += wp[j];
      }
    }
    block_inclusive_scan2_f64<kWThreads>(a, b, lds_d);
    if (threadIdx.x == kWThreads - 1) {
      ws.zres[s * pieces + cp] = a;
      ws.zp[s * pieces + cp] = b;
    }
  }
}

// ---------------------------------------------------------------- sample
template <bool kT>
__global__ __launch_bounds__(kWThreads) void sample_kernel(
    const float* __restrict__ target, const float* __restrict__ draft,
    const float* __restrict__ uniforms, int kd, int v, int pieces, Workspace ws,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ flags, int vec4, Transform tr) {
  __shared__ double lds_scan[kWThreads / kWave];
  __shared__ double s_incl[kWThreads];
  __shared__ int s_fl[2 * kWWaves];
  __shared__ double tab[32];  // visible after the piece selection's barriers
  if (threadIdx.x < 32) tab[threadIdx.x] = kExp2Table32[threadIdx.x];
  const int64_t s = blockIdx.x;
  // the piece totals do not depend on the decision: load them with it
  const bool mine = pieces <= kWThreads && (int)threadIdx.x < pieces;
  const double zres0 = mine ? ws.zres[s * pieces + threadIdx.x] : 0.0;
  const double zp0 = mine ? ws.zp[s * pieces + threadIdx.x] : 0.0;
  const float u_last = uniforms[(size_t)s * (kd + 1) + kd];
  const Decision d = ws.dec[s];
  if (d.n < 0) return;
  FinalRows fr;
  fr.tab = tab;
  fr.ek = exp_consts();
  fr.zt = row_ptr(target, draft, s, kd, d.n, v);
  fr.zd = d.n < kd ? row_ptr(target, draft, s, kd, kd + 1 + d.n, v) : nullptr;
  fr.mt = d.mt;
  fr.inv_st = d.inv_st;
  fr.md = d.md;
  fr.inv_sd = d.inv_sd;
  if constexpr (kT) {
    const int per_seq = 2 * kd + 1;
    fr.inv_tau = tr.inv_tau;
    fr.thr_t = tr.thr ? tr.thr[(size_t)s * per_seq + d.n] : 0u;
    fr.thr_d = (tr.thr && d.n < kd) ? tr.thr[(size_t)s * per_seq + kd + 1 + d.n] : 0u;
    fr.mw = mask_words(tr, s, kd, d.n);
  }
  draw_final<kT>(fr, d.n, kd, v, pieces, s, ws, u_last, out_tokens, flags, vec4, zres0, zp0, lds_scan,
             s_incl, s_fl);
}

// Built-in workspace of spec_accept_noalloc: a file-scope device array, one copy per GPU
// for the life of the process. In host code `scratch` names a host-side stand-in, not the
// device address: every host use goes through the address hipGetSymbolAddress returns.
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // once per device, with that device current (two threads racing here store the same address)
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

namespace {

// The top-k / top-p thresholds of every row into sb.thr, rows = b·(2kd + 1) numbered as
// the stats kernel numbers them; at least one of top-k (sa.top_k > 0) and top-p
// (sa.top_p < 1) is on.
hipError_t launch_selection(const float* target, const float* draft, int32_t b, int32_t kd, int32_t v,
                            const Transform& tr, const SelBufs& sb, const SelArgs& sa_in, const SelStats& ss,
                            bool vec4, hipStream_t stream) {
  const int chunks = (v + kChunk - 1) / kChunk;
  const int64_t rows = (int64_t)b * (2 * kd + 1);
  SelArgs sa = sa_in;
  sa.chunks = chunks;
  sa.slot_log2 = 0;
  if (sa.top_k > 0 && chunks <= kMaxSelChunks) {
    // top-k by per-chunk candidates when k is at most the threads of a chunk's workgroup and
    // 2^c2 >= chunks interleaved shares of 2^lg slots, the smallest power of two (at least 8)
    // holding twice k, fit the list (the finishing workgroup reads only those 2^(c2 + lg))
    int c2 = 0;
    while ((1 << c2) < chunks) ++c2;
    int lg = 3;
    while ((int64_t(1) << lg) < 2 * (int64_t)sa.top_k) ++lg;
    if (sa.top_k <= kThreads && c2 + lg <= kCandLog2) {
      sa.slot_log2 = lg;
      sa.chunk_log2 = c2;
    }
  }
  const dim3 g1((unsigned)rows, (unsigned)chunks);
  if (sa.slot_log2 > 0) {
    if (vec4) sel_chunk_kernel<true><<<g1, dim3(kThreads), 0, stream>>>(target, draft, kd, v, tr, sb, sa);
    else sel_chunk_kernel<false><<<g1, dim3(kThreads), 0, stream>>>(target, draft, kd, v, tr, sb, sa);
    if (vec4)
      sel_finish_kernel<true><<<dim3((unsigned)rows), dim3(kFThreads), 0, stream>>>(target, draft, kd, v, tr, sb, sa, ss);
    else
      sel_finish_kernel<false><<<dim3((unsigned)rows), dim3(kFThreads), 0, stream>>>(target, draft, kd, v, tr, sb, sa, ss);
    return hipGetLastError();
  }
  const bool mass = sa.top_k == 0;  // top-p alone: digit-0 masses in sel_count
  // chunks per counting workgroup: about eight resident workgroups per CU's worth of grid
  const int cpw = (int)std::max<int64_t>(1, std::min<int64_t>(8, rows * chunks / 2048));
  const dim3 gc((unsigned)rows, (unsigned)((chunks + cpw - 1) / cpw));
  sel_clear_kernel<<<dim3((unsigned)rows), dim3(kThreads), 0, stream>>>(sb, mass ? 1 : 0);
  if (vec4 && mass)
    sel_count_kernel<true, true><<<gc, dim3(kThreads), 0, stream>>>(target, draft, kd, v, chunks, cpw, tr, sb, sa);
  else if (vec4)
    sel_count_kernel<true, false><<<gc, dim3(kThreads), 0, stream>>>(target, draft, kd, v, chunks, cpw, tr, sb, sa);
  else if (mass)
    sel_count_kernel<false, true><<<gc, dim3(kThreads), 0, stream>>>(target, draft, kd, v, chunks, cpw, tr, sb, sa);
  else
    sel_count_kernel<false, false><<<gc, dim3(kThreads), 0, stream>>>(target, draft, kd, v, chunks, cpw, tr, sb, sa);
  if (vec4) sel_collect_kernel<true><<<g1, dim3(kThreads), 0, stream>>>(target, draft, kd, v, tr, sb);
  else sel_collect_kernel<false><<<g1, dim3(kThreads), 0, stream>>>(target, draft, kd, v, tr, sb);
  if (vec4)
    sel_finish_kernel<true><<<dim3((unsigned)rows), dim3(kFThreads), 0, stream>>>(target, draft, kd, v, tr, sb, sa, ss);
  else
    sel_finish_kernel<false><<<dim3((unsigned)rows), dim3(kFThreads), 0, stream>>>(target, draft, kd, v, tr, sb, sa, ss);
  return hipGetLastError();
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t value) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

// Selection buffers of `rows` rows carved from a workspace (thresholds elsewhere).
struct SelLayout {
  size_t cnt, mass, state, arrive, rkey, rbad, candn, cand, total;
};
inline SelLayout sel_layout(int64_t rows) {
  SelLayout L;
  size_t off = 0;
  L.cnt = off;
  off = align256(off + sizeof(uint32_t) * rows * kSelB0);
  L.mass = off;
  off = align256(off + sizeof(double) * rows * kSelB0);
  L.state = off;
  off = align256(off + sizeof(SelState) * rows);
  L.arrive = off;
  off = align256(off + sizeof(uint32_t) * rows);
  L.rkey = off;
  off = align256(off + sizeof(uint32_t) * rows);
  L.rbad = off;
  off = align256(off + sizeof(uint32_t) * rows);
  L.candn = off;
  off = align256(off + sizeof(uint32_t) * rows);
  L.cand = off;
  off = align256(off + sizeof(uint32_t) * rows * kCand);
  L.total = off;
  return L;
}

}  // namespace

size_t sampling_thresholds_workspace_bytes(int64_t rows) { return sel_layout(rows).total; }

hipError_t launch_sampling_thresholds(const float* logits, int32_t rows, int32_t v, const SamplingParams& sp,
                                      uint32_t* out_thr, void* workspace, bool vec4, hipStream_t stream) {
  const bool use_k = sp.top_k > 0 && sp.top_k < v;
  const bool use_p = sp.top_p < 1.0f;
  if (!use_k && !use_p) {
    fill_u32_kernel<<<dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream>>>(out_thr, rows, 0u);
    return hipGetLastError();
  }
  Transform tr{};
  tr.mask = sp.mask;
  tr.inv_tau = 1.0 / (double)sp.temperature;
  tr.words = (v + 31) / 32;
  const SelLayout L = sel_layout(rows);
  char* base = static_cast<char*>(workspace);
  SelBufs sb;
  sb.cnt = reinterpret_cast<uint32_t*>(base + L.cnt);
  sb.mass = reinterpret_cast<double*>(base + L.mass);
  sb.state = reinterpret_cast<SelState*>(base + L.state);
  sb.arrive = reinterpret_cast<uint32_t*>(base + L.arrive);
  sb.rkey = reinterpret_cast<uint32_t*>(base + L.rkey);
  sb.candn = reinterpret_cast<uint32_t*>(base + L.candn);
  sb.cand = reinterpret_cast<uint32_t*>(base + L.cand);
  sb.rbad = reinterpret_cast<uint32_t*>(base + L.rbad);
  sb.thr = out_thr;
  const SelArgs sa{use_k ? sp.top_k : 0, use_p ? (double)sp.top_p : 1.0, 0, 0, 0};
  // one "sequence" per row with no draft rows: row s is logits + s·v, mask row s
  return launch_selection(logits, nullptr, rows, 0, v, tr, sb, sa, SelStats{}, vec4, stream);
}

size_t accept_workspace_bytes(int64_t b, int64_t kd, int64_t v, bool sampled) {
  return layout(b, kd, v, sampled).total;
}

hipError_t launch_spec_accept(const float* target, const float* draft, const int32_t* tokens,
                              const float* uniforms, int32_t b, int32_t kd, int32_t v,
                              int32_t* out_tokens, int32_t* out_num, void* workspace,
                              int32_t* flags, bool vec4, const SamplingParams* sp,
                              hipStream_t stream) {
  const int chunks = (v + kChunk - 1) / kChunk;
  const int pieces = (v + kPiece - 1) / kPiece;
  const bool kt = sp != nullptr;
  const Layout L = layout(b, kd, v, kt);
  char* base = static_cast<char*>(workspace);
  Workspace ws;
  ws.cmax = reinterpret_cast<float*>(base + L.cmax);
  ws.csum = reinterpret_cast<double*>(base + L.csum);
  ws.cbad = reinterpret_cast<int32_t*>(base + L.cbad);
  ws.gz = reinterpret_cast<float*>(base + L.gz);
  ws.dec = reinterpret_cast<Decision*>(base + L.dec);
  ws.zres = reinterpret_cast<double*>(base + L.zres);
  ws.zp = reinterpret_cast<double*>(base + L.zp);
  const int64_t rows = (int64_t)b * (2 * kd + 1);
  const dim3 g1((unsigned)rows, (unsigned)chunks);
  hipError_t e = hipSuccess;

  Transform tr{};
  if (kt) {
    tr.mask = sp->mask;
    tr.inv_tau = 1.0 / (double)sp->temperature;
    tr.words = (v + 31) / 32;
    const bool use_k = sp->top_k > 0 && sp->top_k < v;
    const bool use_p = sp->top_p < 1.0f;
    if (use_k || use_p) {
      SelBufs sb;
      sb.cnt = reinterpret_cast<uint32_t*>(base + L.selcnt);
      sb.mass = reinterpret_cast<double*>(base + L.selmass);
      sb.state = reinterpret_cast<SelState*>(base + L.selstate);
      sb.arrive = reinterpret_cast<uint32_t*>(base + L.selarrive);
      sb.rkey = reinterpret_cast<uint32_t*>(base + L.selrkey);
      sb.candn = reinterpret_cast<uint32_t*>(base + L.selcandn);
      sb.cand = reinterpret_cast<uint32_t*>(base + L.selcand);
      sb.thr = reinterpret_cast<uint32_t*>(base + L.thr);
      sb.rbad = reinterpret_cast<uint32_t*>(base + L.selrbad);
      const SelArgs sa{use_k ? sp->top_k : 0, use_p ? (double)sp->top_p : 1.0, 0, 0, 0};
      const SelStats ss{ws.cmax, ws.csum, ws.cbad, ws.gz, reinterpret_cast<uint32_t*>(base + L.sdone), tokens,
                        chunks};
      if ((e = launch_selection(target, draft, b, kd, v, tr, sb, sa, ss, vec4, stream)) != hipSuccess) return e;
      tr.thr = sb.thr;
      tr.sdone = ss.sdone;
    }
  }

  if (vec4 && kt) stats_kernel<true, true><<<g1, dim3(kThreads), 0, stream>>>(target, draft, tokens, kd, v, chunks, ws, tr);
  else if (vec4) stats_kernel<true, false><<<g1, dim3(kThreads), 0, stream>>>(target, draft, tokens, kd, v, chunks, ws, tr);
  else if (kt) stats_kernel<false, true><<<g1, dim3(kThreads), 0, stream>>>(target, draft, tokens, kd, v, chunks, ws, tr);
  else stats_kernel<false, false><<<g1, dim3(kThreads), 0, stream>>>(target, draft, tokens, kd, v, chunks, ws, tr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // prefetch of all candidate rows while the batch's logits are at most 16 MB
  const bool prefetch = (int64_t)b * (2 * kd + 1) * v * 4 <= (int64_t(16) << 20);
  const int per = prefetch ? 1 : 4;  // pieces per workgroup (decide_kernel's kPer)
  const dim3 g2((unsigned)((pieces + per - 1) / per), (unsigned)b);
#define MXS_DECIDE(P, T)                                                                          \
  decide_kernel<P, T><<<g2, dim3(kWThreads), 0, stream>>>(target, draft, tokens, uniforms, kd, v, \
                                                          chunks, pieces, ws, out_tokens, out_num, \
                                                          flags, vec4, tr)
  if (prefetch && kt) MXS_DECIDE(true, true);
  else if (prefetch) MXS_DECIDE(true, false);
  else if (kt) MXS_DECIDE(false, true);
  else MXS_DECIDE(false, false);
#undef MXS_DECIDE
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (kt)
    sample_kernel<true><<<dim3((unsigned)b), dim3(kWThreads), 0, stream>>>(target, draft, uniforms, kd, v,
                                                                           pieces, ws, out_tokens, flags, vec4, tr);
  else
    sample_kernel<false><<<dim3((unsigned)b), dim3(kWThreads), 0, stream>>>(target, draft, uniforms, kd, v,
                                                                            pieces, ws, out_tokens, flags, vec4, tr);
  return hipGetLastError();
}

}  // namespace mxs
