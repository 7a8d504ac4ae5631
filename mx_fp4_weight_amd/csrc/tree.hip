// spec_accept_tree: one verification cycle over a tree of draft tokens per sequence (gfx950).
//
// Rule ("Module 11. Speculative Decoding and Quantization", §4, applied at every node of the
// tree; the lecture's §8 notes that trees verified by typical acceptance lose §4's guarantee):
// a node's children, independent draws from the node's draft law q, are tried in index order;
// child j is accepted with probability min(1, L_j(x)/q(x)), where L_1 = p (the target law of
// the node's history) and, after a rejection, L_{j+1} = norm((L_j - q)+); an accepted child
// becomes the next node; when every child is rejected or the node is a leaf, the final token
// is drawn from the current law by inverse CDF on the supplied uniform. For a chain this is
// spec_accept's rule.
//
// With w_1 = p, Z_1 = 1 and w_{j+1} = (w_j / Z_j - q)+, Z_{j+1} = sum w_{j+1}, the law L_j is
// w_j / Z_j. Kernels on the caller's stream:
//   stats  grid (rows, chunks): chunk max (fp32) and sum exp(z - max) (fp64) of every target
//          and draft row of every node (one full read of the logits).
//   rowstat one workgroup per row: the chunk statistics combined into the row's (max, sum).
//   pass r (r = 0 .. largest child count): grid (pieces, nodes, sequences): for every node
//          with at least r children (r >= 1), the 1024-token piece totals of w_{r+1}, with
//          Z_2 .. Z_r summed from the earlier passes' piece totals in a fixed order; for r = 0
//          the totals of w_1 = p of every leaf (the target row alone). Every node gets them,
//          visited or not: the walk below needs them at once.
//   walk   one workgroup per sequence: walks the tree with scalar decisions (the row statistics
//          are the stored ones and the Z values are summed in the passes' fixed order), then
//          draws the final token: a scan of the final law's piece totals picks the piece, its
//          weights are recomputed exactly as the pass computed them, a scan of the thread
//          totals picks the thread, and its 4 weights give the token.
// Probabilities, laws and prefix sums are fp64.
#include "common.hpp"
#include "internal.hpp"

// No FMA contraction: the walk recomputes a piece's weights bit for bit as the pass did.
#pragma clang fp contract(off)

namespace mxs {
namespace {

constexpr int kTh = 256;           // threads of every tree kernel
constexpr int kSPer = 16;          // logits per thread in the statistics kernel
constexpr int kSChunk = kTh * kSPer;
constexpr int kWPerT = 4;          // tokens per thread of a piece
constexpr int kTPiece = kTh * kWPerT;
constexpr int kWavesT = kTh / kWave;

struct TreeWs {
  float* cmax;    // [b][2(N+1)][chunks]
  double* csum;   // [b][2(N+1)][chunks]
  int32_t* cbad;  // [b][2(N+1)][chunks]
  double* ptot;   // [passes][b][N+1][pieces]: piece totals of w_{r+1}
  double* rms;    // [b][2(N+1)][2]: the row's max and sum exp(z - max)
  int32_t* rbad;  // [b][2(N+1)]: the row is malformed (a NaN / +inf logit, or no finite logit)
};

__device__ inline const float* tree_row(const float* base, int64_t s, int n, int rho, int64_t v) {
  return base + ((size_t)s * (n + 1) + rho) * (size_t)v;
}

// ------------------------------------------------------------------ statistics
// A leaf's draft row (the law its children would be tested against: it has none) is read for
// the malformed-row check alone: its chunks get the maximum and the flag, and a zero sum.
template <bool kVec4>
__global__ __launch_bounds__(kTh) void tree_stats_kernel(const float* __restrict__ target,
                                                        const float* __restrict__ draft, TreeTopo topo, int v,
                                                        int chunks, TreeWs ws) {
  const int n = topo.n;
  __shared__ double lds_d[kWavesT];
  __shared__ float lds_f[kWavesT];
  __shared__ int lds_i[kWavesT];
  __shared__ double tab[32];
  if (threadIdx.x < 32) tab[threadIdx.x] = kExp2Table32[threadIdx.x];
  const int64_t g = blockIdx.x;  // row over all sequences: target rows 0..n, then draft rows 0..n
  const int per = 2 * (n + 1);
  const int64_t s = g / per;
  const int j = (int)(g % per);
  const float* z = j <= n ? tree_row(target, s, n, j, v) : tree_row(draft, s, n, j - n - 1, v);
  const int base = blockIdx.y * kSChunk;
  float vals[kSPer];
  if constexpr (kVec4) {
#pragma unroll
    for (int q = 0; q < kSPer / 4; ++q) {
      const int e = base + 4 * ((int)threadIdx.x + kTh * q);
      f32x4 t = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (e < v) t = *reinterpret_cast<const f32x4*>(z + e);
#pragma unroll
      for (int i = 0; i < 4; ++i) vals[4 * q + i] = t[i];
    }
  } else {
#pragma unroll
    for (int q = 0; q < kSPer; ++q) {
      const int e = base + (int)threadIdx.x + kTh * q;
      vals[q] = e < v ? z[e] : -INFINITY;
    }
  }
  float mx = -INFINITY;
  int bad = 0;
#pragma unroll
  for (int q = 0; q < kSPer; ++q) {
    bad |= (int)nan_or_pinf(vals[q]);
    mx = fmaxf(mx, vals[q]);
  }
  block_max_or<kTh>(mx, bad, lds_f, lds_i);
  const bool leaf_draft = j > n && topo.off[j - n] == topo.off[j - n - 1];  // row j - n - 1 has no children
  double acc = 0.0;
  if (mx != -INFINITY && !bad && !leaf_draft) {
    const double m64 = (double)mx;
    const ExpK ek = exp_consts();
#pragma unroll
    for (int q = 0; q < kSPer; ++q) acc += exp_neg_f64_tab((double)vals[q] - m64, tab, ek);
  }
  acc = block_sum_f64<kTh>(acc, lds_d);
  if (threadIdx.x == 0) {
    const size_t o = (size_t)g * chunks + blockIdx.y;
    ws.cmax[o] = mx;
    ws.csum[o] = acc;
    ws.cbad[o] = bad;
  }
}

// ------------------------------------------------------------------ shared by pass and walk
struct RowStat {
  double m, s;  // max and sum exp(z - max) of the row
  int bad;      // a NaN / +inf logit, or no finite logit
};

// The statistics of row j (0..n target, n+1..2n+1 draft) of sequence s, combined from its
// chunks in a fixed order (every workgroup that needs them gets the same bits). Block-wide.
__device__ RowStat row_stat(const TreeWs& ws, int64_t s, int n, int j, int chunks, double* lds_d, float* lds_f,
                            int* lds_i) {
  const size_t o = ((size_t)s * 2 * (n + 1) + j) * chunks;
  float m = -INFINITY;
  int bad = 0;
  for (int c = threadIdx.x; c < chunks; c += kTh) {
    m = fmaxf(m, ws.cmax[o + c]);
    bad |= ws.cbad[o + c];
  }
  block_max_or<kTh>(m, bad, lds_f, lds_i);
  RowStat r;
  r.m = (double)m;
  r.bad = bad | (m == -INFINITY);
  double sum = 0.0;
  if (!r.bad) {
    for (int c = threadIdx.x; c < chunks; c += kTh) {
      const double cs = ws.csum[o + c];
      if (cs > 0.0) sum += cs * exp_neg_f64((double)ws.cmax[o + c] - r.m);
    }
  }
  r.s = block_sum_f64<kTh>(sum, lds_d);
  return r;
}

// One workgroup per row: its statistics combined once, for the passes and the walk to read.
__global__ __launch_bounds__(kTh) void tree_rowstat_kernel(int n, int chunks, TreeWs ws) {
  __shared__ double lds_d[kWavesT];
  __shared__ float lds_f[kWavesT];
  __shared__ int lds_i[kWavesT];
  const int64_t g = blockIdx.x;
  const int per = 2 * (n + 1);
  const RowStat r = row_stat(ws, g / per, n, (int)(g % per), chunks, lds_d, lds_f, lds_i);
  if (threadIdx.x == 0) {
    ws.rms[2 * g] = r.m;
    ws.rms[2 * g + 1] = r.s;
    ws.rbad[g] = r.bad;
  }
}

__device__ inline RowStat load_stat(const TreeWs& ws, int64_t s, int n, int j) {
  const size_t g = (size_t)s * 2 * (n + 1) + j;
  RowStat r;
  r.m = ws.rms[2 * g];
  r.s = ws.rms[2 * g + 1];
  r.bad = ws.rbad[g];
  return r;
}

// Sum of pass r's piece totals of node rho (Z_{r+1}), in piece order per thread, then the fixed
// block order. Block-wide.
__device__ double pass_sum(const TreeWs& ws, int r, int64_t s, int64_t b, int n, int rho, int pieces, double* lds_d) {
  const double* pt = ws.ptot + (((size_t)r * b + s) * (n + 1) + rho) * pieces;
  double acc = 0.0;
  for (int c = threadIdx.x; c < pieces; c += kTh) acc += pt[c];
  return block_sum_f64<kTh>(acc, lds_d);
}

// w_{r+1} of the 4 tokens t0 .. t0+3 of node rho (0 past v): p, then r residual steps.
struct NodeLaw {
  const float* zt;  // target row of the node
  const float* zd;  // draft row of the node
  double mt, inv_st, md, inv_sd;
  const double* z;  // LDS: z[i] = Z_i for i = 1 .. r (z[1] = 1), the same in every thread
};

__device__ inline void law_weights(const NodeLaw& nl, int r, int t0, int v, bool vec4, const double* tab,
                                   const ExpK& ek, double (&w)[kWPerT]) {
  float zt[kWPerT], zd[kWPerT];
  if (vec4 && t0 + kWPerT <= v) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(nl.zt + t0);
    f32x4 c = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (r > 0) c = *reinterpret_cast<const f32x4*>(nl.zd + t0);  // p alone needs no draft row
#pragma unroll
    for (int j = 0; j < kWPerT; ++j) {
      zt[j] = a[j];
      zd[j] = c[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kWPerT; ++j) {
      const bool in = t0 + j < v;
      zt[j] = in ? nl.zt[t0 + j] : -INFINITY;
      zd[j] = (in && r > 0) ? nl.zd[t0 + j] : -INFINITY;
    }
  }
#pragma unroll
  for (int j = 0; j < kWPerT; ++j) {
    double x = exp_neg_f64_tab((double)zt[j] - nl.mt, tab, ek) * nl.inv_st;
    if (r > 0) {
      const double q = exp_neg_f64_tab((double)zd[j] - nl.md, tab, ek) * nl.inv_sd;
      for (int i = 1; i <= r; ++i) {
        const double d = x / nl.z[i] - q;
        x = d > 0.0 ? d : 0.0;
      }
    }
    w[j] = x;
  }
}

// ------------------------------------------------------------------ residual passes
// ppw pieces per workgroup (consecutive), so large grids stay about one resident round.
template <bool kVec4>
__global__ __launch_bounds__(kTh) void tree_pass_kernel(const float* __restrict__ target,
                                                       const float* __restrict__ draft, TreeTopo topo, int r,
                                                       int v, int pieces, int ppw, int64_t b, TreeWs ws) {
  __shared__ double lds_d[kWavesT];
  __shared__ double tab[32];
  __shared__ double s_z[kMaxTreeChildren + 2];
  if (threadIdx.x < 32) tab[threadIdx.x] = kExp2Table32[threadIdx.x];
  const int n = topo.n;
  const int rho = blockIdx.y;
  const int64_t s = blockIdx.z;
  const int kids = topo.off[rho + 1] - topo.off[rho];
  // uniform: fewer children than tries; and the totals of p (r = 0) only for leaves (an inner
  // node draws from p only after a zero residual, a rounding case the walk covers itself)
  if (r > kids || (r == 0 && kids > 0)) return;
  const RowStat st = load_stat(ws, s, n, rho);
  const RowStat sd = load_stat(ws, s, n, n + 1 + rho);
  double* out = ws.ptot + (((size_t)r * b + s) * (n + 1) + rho) * pieces;
  if (st.bad || sd.bad) {  // the walk refuses the sequence
    for (int i = threadIdx.x; i < ppw; i += kTh)
      if ((int)blockIdx.x * ppw + i < pieces) out[blockIdx.x * ppw + i] = 0.0;
    return;
  }
  NodeLaw nl;
  nl.zt = tree_row(target, s, n, rho, v);
  nl.zd = tree_row(draft, s, n, rho, v);
  nl.mt = st.m;
  nl.inv_st = 1.0 / st.s;
  nl.md = sd.m;
  nl.inv_sd = 1.0 / sd.s;
  if (threadIdx.x == 0) s_z[1] = 1.0;
  for (int i = 2; i <= r; ++i) {
    const double zi = pass_sum(ws, i - 1, s, b, n, rho, pieces, lds_d);
    if (threadIdx.x == 0) s_z[i] = zi;
  }
  __syncthreads();
  nl.z = s_z;
  const ExpK ek = exp_consts();
  for (int i = 0; i < ppw; ++i) {
    const int piece = (int)blockIdx.x * ppw + i;
    if (piece >= pieces) break;  // uniform
    double w[kWPerT];
    law_weights(nl, r, piece * kTPiece + (int)threadIdx.x * kWPerT, v, kVec4, tab, ek, w);
    double t = 0.0;
#pragma unroll
    for (int j = 0; j < kWPerT; ++j) t += w[j];
    t = block_inclusive_scan_f64<kTh>(t, lds_d);
    if (threadIdx.x == kTh - 1) out[piece] = t;
  }
}

// ------------------------------------------------------------------ walk and final draw
constexpr int kNoneT = 0x7fffffff;

// First index with first_cond and last with last_cond over base + threadIdx.x (block-wide).
__device__ inline int2 first_last(bool first_cond, bool last_cond, int base, int* lds) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const unsigned long long m1 = __ballot(first_cond);
  const unsigned long long m2 = __ballot(last_cond);
  if (lane == 0) {
    lds[w] = m1 ? base + w * kWave + __builtin_ctzll(m1) : kNoneT;
    lds[kWavesT + w] = m2 ? base + w * kWave + 63 - __builtin_clzll(m2) : -1;
  }
  __syncthreads();
  int2 res = make_int2(kNoneT, -1);
#pragma unroll
  for (int i = 0; i < kWavesT; ++i) {
    res.x = min(res.x, lds[i]);
    res.y = max(res.y, lds[kWavesT + i]);
  }
  __syncthreads();
  return res;
}

template <bool kVec4>
__global__ __launch_bounds__(kTh) void tree_walk_kernel(const float* __restrict__ target,
                                                       const float* __restrict__ draft,
                                                       const int32_t* __restrict__ tokens,
                                                       const float* __restrict__ uniforms, TreeTopo topo, int v,
                                                       int chunks, int pieces, int64_t b, TreeWs ws,
                                                       int32_t* __restrict__ out_tokens,
                                                       int32_t* __restrict__ out_nodes,
                                                       int32_t* __restrict__ out_num, int32_t* __restrict__ flags) {
  __shared__ double lds_d[kWavesT];
  __shared__ int lds_i[kWavesT];
  __shared__ int s_fl[2 * kWavesT];
  __shared__ double s_incl[kTh];
  __shared__ double tab[32];
  __shared__ double s_z[kMaxTreeChildren + 2];
  __shared__ int s_move;
  if (threadIdx.x < 32) tab[threadIdx.x] = kExp2Table32[threadIdx.x];
  const int n = topo.n;
  const int64_t s = blockIdx.x;
  int32_t* ot = out_tokens + (size_t)s * (topo.depth + 1);
  int32_t* on = out_nodes + (size_t)s * topo.depth;

  // every row of the tree is examined: a malformed one refuses the sequence
  int bad = 0;
  for (int j = threadIdx.x; j < 2 * (n + 1); j += kTh) bad |= ws.rbad[(size_t)s * 2 * (n + 1) + j];
  bad = block_or<kTh>(bad, lds_i);
  for (int i = threadIdx.x; i <= topo.depth; i += kTh) {
    ot[i] = -1;
    if (i < topo.depth) on[i] = -1;
  }
  if (bad) {
    if (threadIdx.x == 0) {
      out_num[s] = 0;
      raise_flag(flags, MXS_FLAG_NONFINITE);
    }
    return;
  }

  int rho = 0;  // the current node's row (0: the root)
  int nacc = 0;
  int f = 1;    // the final law L_f of the node where the walk stops
  int fl = 0;
  NodeLaw nl;
  while (true) {
    const RowStat st = load_stat(ws, s, n, rho);
    const RowStat sd = load_stat(ws, s, n, n + 1 + rho);
    nl.zt = tree_row(target, s, n, rho, v);
    nl.zd = tree_row(draft, s, n, rho, v);
    nl.mt = st.m;
    nl.inv_st = 1.0 / st.s;
    nl.md = sd.m;
    nl.inv_sd = 1.0 / sd.s;
    nl.z = s_z;
    if (threadIdx.x == 0) s_z[1] = 1.0;
    const int c0 = topo.off[rho], m = topo.off[rho + 1] - c0;
    int moved = -1;
    f = 1;
    for (int j = 1; j <= m; ++j) {
      const int c = topo.child[c0 + j - 1];
      if (threadIdx.x == 0) {
        const int x = tokens[(size_t)s * n + c];
        double a = 0.0;
        if (x < 0 || x >= v) {
          fl |= MXS_FLAG_TOKEN_RANGE;
        } else {
          const double q = exp_neg_f64((double)nl.zd[x] - nl.md) / sd.s;
          double w = exp_neg_f64((double)nl.zt[x] - nl.mt) / st.s;
          for (int i = 1; i < j; ++i) {
            const double d = w / nl.z[i] - q;
            w = d > 0.0 ? d : 0.0;
          }
          if (q == 0.0) {
            fl |= MXS_FLAG_Q_ZERO;
          } else {
            a = (w / nl.z[j]) / q;
            a = a < 1.0 ? a : 1.0;
          }
        }
        const float u = uniforms[(size_t)s * (n + 1) + c];
        s_move = (double)u < a ? c : -1;
      }
      __syncthreads();
      moved = s_move;
      __syncthreads();
      if (moved >= 0) break;
      // rejected: the next law L_{j+1} needs Z_{j+1} (pass j's total for this node)
      const double znext = pass_sum(ws, j, s, b, n, rho, pieces, lds_d);
      if (threadIdx.x == 0) s_z[j + 1] = znext;
      __syncthreads();
      if (!(znext > 0.0)) {  // no residual mass (rounding): draw from L_j, try no further child
        fl |= MXS_FLAG_RESIDUAL_ZERO;
        f = j;
        break;
      }
      f = j + 1;
    }
    if (moved < 0) break;
    if (threadIdx.x == 0) {
      ot[nacc] = tokens[(size_t)s * n + moved];
      on[nacc] = moved;
    }
    ++nacc;
    rho = moved + 1;
  }

  // final token from L_f = w_f / Z_f of row rho by inverse CDF: the piece, then the thread,
  // then the token
  double* ptw = ws.ptot + (((size_t)(f - 1) * b + s) * (n + 1) + rho) * pieces;
  const ExpK ek = exp_consts();
  if (f == 1 && topo.off[rho + 1] > topo.off[rho]) {
    // an inner node drawing from p (after a zero residual): the pass left its totals of p out,
    // so this workgroup computes them, piece by piece, exactly as the pass computes them
    for (int pc = 0; pc < pieces; ++pc) {
      double w[kWPerT];
      law_weights(nl, 0, pc * kTPiece + (int)threadIdx.x * kWPerT, v, kVec4, tab, ek, w);
      double t = 0.0;
#pragma unroll
      for (int j = 0; j < kWPerT; ++j) t += w[j];
      t = block_inclusive_scan_f64<kTh>(t, lds_d);
      if (threadIdx.x == kTh - 1) ptw[pc] = t;
    }
    __syncthreads();
  }
  const double* pt = ptw;
  const float u = uniforms[(size_t)s * (n + 1) + n];
  double zsum = 0.0;
  for (int c0 = 0; c0 < pieces; c0 += kTh) {
    const int cc = c0 + (int)threadIdx.x;
    zsum += block_sum_f64<kTh>(cc < pieces ? pt[cc] : 0.0, lds_d);
  }
  const double uz = (double)u * zsum;
  int piece = kNoneT, lastp = -1;
  double before = 0.0, carry = 0.0;
  for (int c0 = 0; c0 < pieces && piece == kNoneT; c0 += kTh) {
    const int cc = c0 + (int)threadIdx.x;
    const double zc = cc < pieces ? pt[cc] : 0.0;
    const double incl = carry + block_inclusive_scan_f64<kTh>(zc, lds_d);
    s_incl[threadIdx.x] = incl;
    const bool pos = cc < pieces && zc > 0.0;
    const int2 q = first_last(pos && uz < incl, pos, c0, s_fl);
    lastp = max(lastp, q.y);
    if (q.x != kNoneT) {
      piece = q.x;
      before = piece > c0 ? s_incl[piece - c0 - 1] : carry;
    }
    carry = s_incl[kTh - 1];
    __syncthreads();
  }
  const bool found = piece != kNoneT;
  if (!found) piece = lastp;  // no crossing (rounding): the last piece with positive weight
  if (piece >= 0) {
    const int t0 = piece * kTPiece + (int)threadIdx.x * kWPerT;
    double w[kWPerT];
    law_weights(nl, f - 1, t0, v, kVec4, tab, ek, w);
    double tt = 0.0;
#pragma unroll
    for (int j = 0; j < kWPerT; ++j) tt += w[j];
    const double sincl = block_inclusive_scan_f64<kTh>(tt, lds_d);
    s_incl[threadIdx.x] = sincl;
    const bool pos = tt > 0.0;
    const int2 q = first_last(pos && found && uz < before + sincl, pos, 0, s_fl);
    const int ti = q.x != kNoneT ? q.x : q.y;
    if ((int)threadIdx.x == ti) {
      const double base = before + (ti > 0 ? s_incl[ti - 1] : 0.0);
      double run = 0.0;
      int pick = -1, lastpos = -1;
#pragma unroll
      for (int j = 0; j < kWPerT; ++j) {
        run += w[j];
        if (w[j] > 0.0) lastpos = t0 + j;
        if (found && pick < 0 && w[j] > 0.0 && uz < base + run) pick = t0 + j;
      }
      ot[nacc] = pick >= 0 ? pick : lastpos;
    }
  }
  if (threadIdx.x == 0) {
    out_num[s] = nacc;
    if (fl) raise_flag(flags, fl);
  }
}

inline size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

size_t tree_workspace_bytes(int64_t b, const TreeTopo& topo, int64_t v) {
  const int64_t rows = b * 2 * (topo.n + 1);
  const int64_t chunks = (v + kSChunk - 1) / kSChunk;
  const int64_t pieces = (v + kTPiece - 1) / kTPiece;
  size_t off = 0;
  off = al256(off + sizeof(float) * rows * chunks);
  off = al256(off + sizeof(double) * rows * chunks);
  off = al256(off + sizeof(int32_t) * rows * chunks);
  off = al256(off + sizeof(double) * (size_t)topo.passes * b * (topo.n + 1) * pieces);
  off = al256(off + sizeof(double) * 2 * rows);
  off = al256(off + sizeof(int32_t) * rows);
  return off;
}

hipError_t launch_spec_accept_tree(const float* target, const float* draft, const TreeTopo& topo,
                                   const int32_t* tokens, const float* uniforms, int32_t b, int32_t v,
                                   int32_t* out_tokens, int32_t* out_nodes, int32_t* out_num, void* workspace,
                                   int32_t* flags, bool vec4, hipStream_t stream) {
  const int n = topo.n;
  const int64_t rows = (int64_t)b * 2 * (n + 1);
  const int chunks = (v + kSChunk - 1) / kSChunk;
  const int pieces = (v + kTPiece - 1) / kTPiece;
  char* base = static_cast<char*>(workspace);
  TreeWs ws;
  size_t off = 0;
  ws.cmax = reinterpret_cast<float*>(base + off);
  off = al256(off + sizeof(float) * rows * chunks);
  ws.csum = reinterpret_cast<double*>(base + off);
  off = al256(off + sizeof(double) * rows * chunks);
  ws.cbad = reinterpret_cast<int32_t*>(base + off);
  off = al256(off + sizeof(int32_t) * rows * chunks);
  ws.ptot = reinterpret_cast<double*>(base + off);
  off = al256(off + sizeof(double) * (size_t)topo.passes * b * (n + 1) * pieces);
  ws.rms = reinterpret_cast<double*>(base + off);
  off = al256(off + sizeof(double) * 2 * rows);
  ws.rbad = reinterpret_cast<int32_t*>(base + off);
  if (vec4)
    tree_stats_kernel<true><<<dim3((unsigned)rows, (unsigned)chunks), dim3(kTh), 0, stream>>>(target, draft, topo, v,
                                                                                             chunks, ws);
  else
    tree_stats_kernel<false><<<dim3((unsigned)rows, (unsigned)chunks), dim3(kTh), 0, stream>>>(target, draft, topo,
                                                                                              v, chunks, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  tree_rowstat_kernel<<<dim3((unsigned)rows), dim3(kTh), 0, stream>>>(n, chunks, ws);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // four pieces per workgroup once one piece each would take several resident rounds
  const int ppw = (int64_t)pieces * (n + 1) * b > 16384 ? 4 : 1;
  for (int r = 0; r < topo.passes; ++r) {
    const dim3 grid((unsigned)((pieces + ppw - 1) / ppw), (unsigned)(n + 1), (unsigned)b);
    if (vec4)
      tree_pass_kernel<true><<<grid, dim3(kTh), 0, stream>>>(target, draft, topo, r, v, pieces, ppw, b, ws);
    else
      tree_pass_kernel<false><<<grid, dim3(kTh), 0, stream>>>(target, draft, topo, r, v, pieces, ppw, b, ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (vec4)
    tree_walk_kernel<true><<<dim3((unsigned)b), dim3(kTh), 0, stream>>>(target, draft, tokens, uniforms, topo, v,
                                                                       chunks, pieces, b, ws, out_tokens, out_nodes,
                                                                       out_num, flags);
  else
    tree_walk_kernel<false><<<dim3((unsigned)b), dim3(kTh), 0, stream>>>(target, draft, tokens, uniforms, topo, v,
                                                                        chunks, pieces, b, ws, out_tokens, out_nodes,
                                                                        out_num, flags);
  return hipGetLastError();
}

}  // namespace mxs
