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
// The fp64 exponentials bound decide and sample at small batches, so their
// pieces are small: many workgroups share the work of one sequence.
// All probabilities and prefix sums are fp64; the result can differ from an
// exact-arithmetic draw only when u_K·Z lies within ~1e-15·Z of an interval
// end. Rounding guards: if no crossing is found where the level above
// placed it, the last positive-weight token of that range is taken, so a
// zero-weight token is never returned.
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
  size_t thr, selmax, selcnt, selmass, selstate, selarrive;
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
    constexpr size_t kBuckets = 2048, kStateBytes = 32;
    L.thr = off;
    off = align256(off + sizeof(uint32_t) * rows);
    L.selmax = off;
    off = align256(off + sizeof(float) * rows * chunks);
    L.selcnt = off;
    off = align256(off + sizeof(uint32_t) * rows * kBuckets);
    L.selmass = off;
    off = align256(off + sizeof(double) * rows * kBuckets);
    L.selstate = off;
    off = align256(off + kStateBytes * rows);
    L.selarrive = off;
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
  // the logit of this row's draft token x (target row i < kd or draft row i), if it is in this chunk
  int xi = -1;
  if (j < kd) xi = tokens[(size_t)s * kd + j];
  else if (j > kd) xi = tokens[(size_t)s * kd + (j - kd - 1)];
  float mx = -INFINITY;
  int bad = 0;
  const uint32_t* mw = nullptr;
  uint32_t thr = 0u;
  if constexpr (kT) {
    mw = mask_words(tr, s, kd, mask_row(j, kd));
    thr = tr.thr ? tr.thr[rowg] : 0u;
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
    bad |= (vals[q] != vals[q]) | (vals[q] == INFINITY);
    const int e = kVec4 ? base + 4 * (threadIdx.x + kThreads * (q / 4)) + (q % 4)
                        : base + threadIdx.x + kThreads * q;
    if constexpr (kT) {
      const bool ok = ((words[q] >> (e & 31)) & 1u) && order_key(vals[q]) >= thr;
      vals[q] = ok ? vals[q] : -INFINITY;
    }
    mx = fmaxf(mx, vals[q]);
    if (e == xi) ws.gz[rowg] = vals[q];
  }
  block_max_or<kThreads>(mx, bad, lds_f, lds_i);
  double acc = 0.0;
  if (mx != -INFINITY && !bad) {
    const double m64 = (double)mx;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      if constexpr (kT) acc += exp_neg_f64_tab(((double)vals[q] - m64) * tr.inv_tau, tab);
      else acc += exp_neg_f64_tab((double)vals[q] - m64, tab);
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
    const double p = exp_neg_f64_tab(dt, fr.tab) * fr.inv_st;
    wp[j] = p;
    if (fr.zd) {
      const double dd = kT ? ((double)zd[j] - fr.md) * fr.inv_tau : (double)zd[j] - fr.md;
      const double q = exp_neg_f64_tab(dd, fr.tab) * fr.inv_sd;
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
// A row's threshold is an order key: a token stays iff its key is at least the
// threshold. Both selections are radix walks over the 32-bit keys of the allowed
// finite logits, top digit (11 bits) first, bottom digit (10 bits) last. A pass over
// the row histograms the current digit of the tokens whose higher digits equal the
// prefix found so far (counts for top-k; counts and fp64 masses exp((z - max) / tau)
// of the tokens top-k kept, for top-p), each workgroup in LDS, then added into the
// row's histogram in the workspace. The last workgroup of the row to finish walks
// that histogram from the largest key down and takes the lowest non-empty bucket
// whose tokens still have fewer than k tokens (top-k) or less than P·S mass (top-p)
// strictly above them; its digit extends the prefix. It then clears the histogram
// and the arrival counter for the next pass. After the last digit the prefix is the
// row's threshold.
constexpr int kSelBuckets = 2048;
constexpr int kSelDigits = 3;
__host__ __device__ constexpr int sel_shift(int d) { return d == 0 ? 21 : (d == 1 ? 10 : 0); }
__host__ __device__ constexpr int sel_width(int d) { return d == 2 ? 10 : 11; }

struct SelState {
  uint32_t prefix;  // resolved key digits (key >> shift of the last resolved digit)
  uint32_t thr_k;   // top-k threshold once resolved (0: top-k off)
  double carry;     // count (top-k) or mass (top-p) strictly above the prefix's key range
  double s1;        // top-p: mass of the law top-k left
  float rmax;       // largest allowed finite logit of the row
  int empty;        // no allowed finite logit (or nothing to select): threshold 0
};

struct SelBufs {
  uint32_t* cnt;     // [rows][kSelBuckets]
  double* mass;      // [rows][kSelBuckets]
  SelState* state;   // [rows]
  uint32_t* arrive;  // [rows] workgroups of the current pass that have finished
  float* cmax;       // [rows][chunks] chunk maxima of the allowed finite logits
  uint32_t* thr;     // [rows] output thresholds
};

struct SelArgs {
  int top_k;     // 0: off
  double top_p;  // >= 1: off
};
static_assert(sizeof(SelState) == 32, "workspace layout assumes a 32-byte selection state");

// The allowed logits of this thread's 16 tokens of a chunk (removed ones: NaN), in the
// stats kernel's order.
template <bool kVec4>
__device__ inline void chunk_logits(const float* __restrict__ z, const uint32_t* mw, int base, int v,
                                    float (&vals)[kPer]) {
#pragma unroll
  for (int q = 0; q < kPer; ++q) vals[q] = NAN;
  if constexpr (kVec4) {
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const int e = base + 4 * ((int)threadIdx.x + kThreads * q);
      if (e < v) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(z + e);
        const uint32_t w = mw ? mw[e >> 5] : 0xFFFFFFFFu;  // the 4 tokens share one mask word
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = ((w >> ((e + i) & 31)) & 1u) && t[i] > -INFINITY && t[i] < INFINITY;
          vals[4 * q + i] = ok ? t[i] : NAN;
        }
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = base + (int)threadIdx.x + kThreads * q;
      if (e < v) {
        const float t = z[e];
        const bool ok = (mw ? ((mw[e >> 5] >> (e & 31)) & 1u) != 0u : true) && t > -INFINITY && t < INFINITY;
        vals[q] = ok ? t : NAN;
      }
    }
  }
}

// Walk the histogram of `digit` (mode 0: counts against k; mode 1: masses against P·S)
// and extend st.prefix with the boundary bucket. Every thread returns the same state.
// The histogram was filled by atomics of other workgroups of the same launch: it is
// read with agent-scope atomic loads.
__device__ void sel_resolve(int mode, int digit, uint32_t* cnt, double* mass, const SelArgs& sa,
                            SelState& st,
                            double* lds_scan, double* s_excl, int* s_fl, int* s_best,
                            double* s_above) {
  const int nb = 1 << sel_width(digit);
  const int per = nb / kThreads;  // 8 or 4 buckets per thread, in descending key order
  const int tid = threadIdx.x;
  uint32_t c[8];
  double w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int b = nb - 1 - (tid * per + i);
    c[i] = i < per ? __hip_atomic_load(&cnt[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    const double m = (i < per && mode == 1)
                         ? __hip_atomic_load(&mass[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : 0.0;
    w[i] = i < per ? (mode == 0 ? (double)c[i] : m) : 0.0;
  }
  if (mode == 1 && digit == 0) {
    // S: the mass of every token top-k kept (all buckets of the first top-p digit)
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) t += w[i];
    st.s1 = block_sum_f64<kThreads>(t, lds_scan);
  }
  const double target = mode == 0 ? (double)sa.top_k : sa.top_p * st.s1;
  double local = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) local += w[i];
  const double incl = block_inclusive_scan_f64<kThreads>(local, lds_scan);
  s_excl[tid] = incl;
  __syncthreads();
  double run = st.carry + (tid > 0 ? s_excl[tid - 1] : 0.0);
  int best = -1;
  double best_above = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i < per && run < target && c[i] > 0u) {
      best = tid * per + i;
      best_above = run;
    }
    run += w[i];
  }
  // descending indices grow with the thread index: the last thread with a candidate
  // holds the lowest qualifying bucket
  const int2 fl = block_first_last(false, best >= 0, 0, s_fl);
  if (tid == fl.y) {
    *s_best = best;
    *s_above = best_above;
  }
  __syncthreads();
  if (fl.y < 0) {
    st.empty = 1;
  } else {
    st.prefix = (st.prefix << sel_width(digit)) | (uint32_t)(nb - 1 - *s_best);
    st.carry = *s_above;
  }
  __syncthreads();
}

// Chunk maxima of the allowed finite logits; clears the row's histogram and counter.
template <bool kVec4>
__global__ __launch_bounds__(kThreads) void sel_prep_kernel(const float* __restrict__ target,
                                                            const float* __restrict__ draft, int kd,
                                                            int v, int chunks, Transform tr,
                                                            SelBufs sb) {
  __shared__ float lds_f[kThreads / kWave];
  const int64_t rowg = blockIdx.x;
  const int per_seq = 2 * kd + 1;
  const int64_t s = rowg / per_seq;
  const int j = (int)(rowg % per_seq);
  const int c = blockIdx.y;
  float vals[kPer];
  chunk_logits<kVec4>(row_ptr(target, draft, s, kd, j, v), mask_words(tr, s, kd, mask_row(j, kd)),
                      c * kChunk, v, vals);
  float mx = -INFINITY;
#pragma unroll
  for (int q = 0; q < kPer; ++q) mx = fmaxf(mx, vals[q]);  // NaN (removed) is ignored
  mx = block_max<kThreads>(mx, lds_f);
  if (threadIdx.x == 0) sb.cmax[rowg * chunks + c] = mx;
  for (int b = c * kThreads + (int)threadIdx.x; b < kSelBuckets; b += chunks * kThreads) {
    sb.cnt[rowg * kSelBuckets + b] = 0u;
    sb.mass[rowg * kSelBuckets + b] = 0.0;
  }
  if (c == 0 && threadIdx.x == 0) sb.arrive[rowg] = 0u;
}

// One pass of the walk: histogram (mode, digit) over this chunk into the row's
// histogram; the row's last workgroup resolves the digit (and at the end of the walk
// writes the threshold).
template <bool kVec4>
__global__ __launch_bounds__(kThreads) void sel_pass_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, int kd, int v, int chunks,
    Transform tr, SelBufs sb, SelArgs sa, int first, int mode, int digit, int last) {
  __shared__ uint32_t hc[kSelBuckets];
  __shared__ double hm[kSelBuckets];
  __shared__ double lds_scan[kThreads / kWave];
  __shared__ double s_excl[kThreads];
  __shared__ float lds_f[kThreads / kWave];
  __shared__ int s_fl[2 * (kThreads / kWave)];
  __shared__ int s_best, s_last_wg;
  __shared__ double s_above;
  const int64_t rowg = blockIdx.x;
  const int per_seq = 2 * kd + 1;
  const int64_t s = rowg / per_seq;
  const int j = (int)(rowg % per_seq);
  const int c = blockIdx.y;
  const int tid = threadIdx.x;

  float vals[kPer];
  chunk_logits<kVec4>(row_ptr(target, draft, s, kd, j, v), mask_words(tr, s, kd, mask_row(j, kd)),
                      c * kChunk, v, vals);

  SelState st;
  if (first) {
    float m = -INFINITY;
    for (int cc = tid; cc < chunks; cc += kThreads) m = fmaxf(m, sb.cmax[rowg * chunks + cc]);
    m = block_max<kThreads>(m, lds_f);
    st.prefix = 0u;
    st.thr_k = 0u;
    st.carry = 0.0;
    st.s1 = 0.0;
    st.rmax = m;
    st.empty = m == -INFINITY;
  } else {
    st = sb.state[rowg];
  }

  const int nb = 1 << sel_width(digit);
  for (int b = tid; b < nb; b += kThreads) {
    hc[b] = 0u;
    hm[b] = 0.0;
  }
  __syncthreads();
  if (!st.empty) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const float zq = vals[q];
      if (zq != zq) continue;  // removed, non-finite or past the row
      const uint32_t key = order_key(zq);
      if (mode == 1 && key < st.thr_k) continue;
      if (digit > 0 && (key >> sel_shift(digit - 1)) != st.prefix) continue;
      const int b = (int)((key >> sel_shift(digit)) & (uint32_t)(nb - 1));
      atomicAdd(&hc[b], 1u);
      if (mode == 1) atomicAdd(&hm[b], exp_neg_f64(((double)zq - (double)st.rmax) * tr.inv_tau));
    }
  }
  __syncthreads();
  uint32_t* gc = sb.cnt + rowg * kSelBuckets;
  double* gm = sb.mass + rowg * kSelBuckets;
  for (int b = tid; b < nb; b += kThreads) {
    if (hc[b] != 0u) {
      atomicAdd(&gc[b], hc[b]);
      if (mode == 1) atomicAdd(&gm[b], hm[b]);
    }
  }
  // arrival. The additions are device-scope atomics, performed where every CU reads them
  // with device-scope loads; each wave waits until its own have completed, so the count
  // cannot run ahead of them. No plain store is shared, so no L2 write-back is needed: a
  // release / acquire fence pair here (an L2 write-back and invalidation in every
  // workgroup) measured 0.7 -> 10.7 ms for top-k + top-p at B = 64.
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  __syncthreads();
  if (tid == 0) {
    const uint32_t before = __hip_atomic_fetch_add(&sb.arrive[rowg], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    s_last_wg = before == (uint32_t)(chunks - 1);
  }
  __syncthreads();
  if (!s_last_wg) return;

  // the row's last workgroup: resolve this digit from the complete histogram
  if (!st.empty) sel_resolve(mode, digit, gc, gm, sa, st, lds_scan, s_excl, s_fl, &s_best, &s_above);
  const bool k_done = mode == 0 && digit == kSelDigits - 1;
  if (k_done) {
    st.thr_k = st.empty ? 0u : st.prefix;  // top-k resolved; a top-p walk starts afresh
    st.prefix = 0u;
    st.carry = 0.0;
  }
  for (int b = tid; b < nb; b += kThreads) {
    gc[b] = 0u;
    gm[b] = 0.0;
  }
  if (tid == 0) {
    sb.arrive[rowg] = 0u;
    sb.state[rowg] = st;
    if (last) sb.thr[rowg] = st.empty ? 0u : (k_done ? st.thr_k : st.prefix);
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
#pragma unroll
  for (int pc = 0; pc < kPer; ++pc) {
    const int cp = c * kPer + pc;  // this piece (uniform: the loop holds block scans)
    if (cp >= pieces) break;
    const int t0p = cp * kPiece + threadIdx.x * kWPer;
    double a = 0.0, b = 0.0;
    FinalRows fr;
    fr.tab = tab;
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
      sb.cmax = reinterpret_cast<float*>(base + L.selmax);
      sb.thr = reinterpret_cast<uint32_t*>(base + L.thr);
      const SelArgs sa{use_k ? sp->top_k : 0, use_p ? (double)sp->top_p : 1.0};
      if (vec4) sel_prep_kernel<true><<<g1, dim3(kThreads), 0, stream>>>(target, draft, kd, v, chunks, tr, sb);
      else sel_prep_kernel<false><<<g1, dim3(kThreads), 0, stream>>>(target, draft, kd, v, chunks, tr, sb);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      // passes: the top-k digits, then the top-p digits
      const int npass = kSelDigits * ((use_k ? 1 : 0) + (use_p ? 1 : 0));
      int h = 0;
      for (int mode = 0; mode < 2; ++mode) {
        if ((mode == 0 && !use_k) || (mode == 1 && !use_p)) continue;
        for (int d = 0; d < kSelDigits; ++d, ++h) {
          const int first = h == 0, last = h == npass - 1;
          if (vec4)
            sel_pass_kernel<true><<<g1, dim3(kThreads), 0, stream>>>(target, draft, kd, v, chunks, tr, sb,
                                                                     sa, first, mode, d, last);
          else
            sel_pass_kernel<false><<<g1, dim3(kThreads), 0, stream>>>(target, draft, kd, v, chunks, tr, sb,
                                                                      sa, first, mode, d, last);
          if ((e = hipGetLastError()) != hipSuccess) return e;
        }
      }
      uint32_t* thr = sb.thr;
      tr.thr = thr;
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
