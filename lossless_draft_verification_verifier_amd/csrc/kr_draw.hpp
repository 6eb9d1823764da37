// kr_draw.hpp -- the replacement / bonus draw in fp64.
//
// After the first rejection at position L the replacement token comes from the
// normalised residual max(0, p - q) of row pair (k*, L) (SpecDiff-2 section 2;
// DiffuSpec section 3, "Acceptance and rejection"); when every drafted token
// is accepted the bonus token comes from p of row gamma.  A residual without
// mass (p equal to q in double) falls back to p.  The token is the first one
// whose cumulative weight exceeds t = u * Z, so tokens of zero weight are
// never drawn; if rounding leaves no such token, the last token with weight.
//
// The drawn rows are recomputed from the logits in fp64, in three launches:
//
// kr_draw_pass (prefix, vocabulary segment of kDrawSeg tokens), one fp64 pass:
//   residual draw: with the exact row maxima from the row-statistics kernel,
//     w_p = exp(z_p/T_p - M_p) and w_q likewise; the segment sums of w_p and
//     w_q give the exact normalisers S_p, S_q.  Whether p_v > q_v, i.e.
//     w_p > (S_p/S_q) w_q, is decided against the fp32 ratio from the
//     row-statistics kernel with a relative margin kClassMargin far above its
//     error: sure-positive tokens add w_p and w_q to two more segment sums, so
//     sum_v max(0, p_v - q_v) over them is (sum w_p)/S_p - (sum w_q)/S_q;
//     tokens inside the margin (a few per row) are stored with their exact
//     weights and settled once S_p and S_q are known.
//   bonus draw: segment max, then the sum of exp(z/T - m_seg).
// kr_draw_fix (prefix, segment): a segment whose list of uncertain tokens
//   overflowed (a cluster of equal p/q ratios, which bf16 logits make
//   possible) gets its residual mass recomputed exactly, in parallel.
// kr_draw_pick (prefix): exact normalisers and per-segment masses, the
//   segment that holds t, then each thread takes kRun consecutive tokens of
//   that segment into registers, and a workgroup prefix sum over the threads'
//   totals locates the token.
// Every reduction has a fixed order and the uncertain tokens are summed in
// token order, so the result is deterministic.
#pragma once

#include "svd_device.hpp"

namespace svd {

constexpr int kUncCap = 32;            // uncertain tokens kept per segment
constexpr int kPickSegs = 256;         // segment records the pick stages in LDS
constexpr double kClassMargin = 2e-4;  // relative margin of the p > q test

// ---------------------------------------------------------------------------
// exp(x) in fp64 for x <= 0 (a few ulp above 0 is fine; x must not be NaN):
// x = n ln2/64 + r with |r| <= ln2/128 (Cody-Waite split of ln2/64; n ln2_hi
// is exact for |n| < 2^17), exp(r) by its degree-5 Taylor polynomial (the
// next term is below 4e-17), 2^(j/64) from a 64-entry table, then ldexp.

struct Exp64Table {
  double t[64];
};

// 2^(j/64), j = 0..63, correctly rounded to double.
__constant__ double kExp2Frac64[64] = {
    0x1.0000000000000p+0, 0x1.02c9a3e778061p+0, 0x1.059b0d3158574p+0, 0x1.0874518759bc8p+0,
    0x1.0b5586cf9890fp+0, 0x1.0e3ec32d3d1a2p+0, 0x1.11301d0125b51p+0, 0x1.1429aaea92de0p+0,
    0x1.172b83c7d517bp+0, 0x1.1a35beb6fcb75p+0, 0x1.1d4873168b9aap+0, 0x1.2063b88628cd6p+0,
    0x1.2387a6e756238p+0, 0x1.26b4565e27cddp+0, 0x1.29e9df51fdee1p+0, 0x1.2d285a6e4030bp+0,
    0x1.306fe0a31b715p+0, 0x1.33c08b26416ffp+0, 0x1.371a7373aa9cbp+0, 0x1.3a7db34e59ff7p+0,
    0x1.3dea64c123422p+0, 0x1.4160a21f72e2ap+0, 0x1.44e086061892dp+0, 0x1.486a2b5c13cd0p+0,
    0x1.4bfdad5362a27p+0, 0x1.4f9b2769d2ca7p+0, 0x1.5342b569d4f82p+0, 0x1.56f4736b527dap+0,
    0x1.5ab07dd485429p+0, 0x1.5e76f15ad2148p+0, 0x1.6247eb03a5585p+0, 0x1.6623882552225p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6dfb23c651a2fp+0, 0x1.71f75e8ec5f74p+0, 0x1.75feb564267c9p+0,
    0x1.7a11473eb0187p+0, 0x1.7e2f336cf4e62p+0, 0x1.82589994cce13p+0, 0x1.868d99b4492edp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8f1ae99157736p+0, 0x1.93737b0cdc5e5p+0, 0x1.97d829fde4e50p+0,
    0x1.9c49182a3f090p+0, 0x1.a0c667b5de565p+0, 0x1.a5503b23e255dp+0, 0x1.a9e6b5579fdbfp+0,
    0x1.ae89f995ad3adp+0, 0x1.b33a2b84f15fbp+0, 0x1.b7f76f2fb5e47p+0, 0x1.bcc1e904bc1d2p+0,
    0x1.c199bdd85529cp+0, 0x1.c67f12e57d14bp+0, 0x1.cb720dcef9069p+0, 0x1.d072d4a07897cp+0,
    0x1.d5818dcfba487p+0, 0x1.da9e603db3285p+0, 0x1.dfc97337b9b5fp+0, 0x1.e502ee78b3ff6p+0,
    0x1.ea4afa2a490dap+0, 0x1.efa1bee615a27p+0, 0x1.f50765b6e4540p+0, 0x1.fa7c1819e90d8p+0,
};

__device__ __forceinline__ void exp64_table_init(Exp64Table &tab) {
  if (threadIdx.x < 64) tab.t[threadIdx.x] = kExp2Frac64[threadIdx.x];
}

__device__ __forceinline__ double exp_nonpos(double x, const Exp64Table &tab) {
  x = fmax(x, -760.0);  // exp(-760) is 0 in double; also maps -inf
  const double n = __builtin_rint(x * 92.33248261689366);  // 64 / ln 2
  const int ni = (int)n;
  double r = __builtin_fma(-n, 0x1.62e42fefa0000p-7, x);
  r = __builtin_fma(-n, 0x1.cf79abc9e3b3ap-46, r);
  double p = 1.0 / 120.0;
  p = __builtin_fma(p, r, 1.0 / 24.0);
  p = __builtin_fma(p, r, 1.0 / 6.0);
  p = __builtin_fma(p, r, 0.5);
  p = __builtin_fma(p, r, 1.0);
  p = __builtin_fma(p, r, 1.0);
  return ldexp(tab.t[ni & 63] * p, ni >> 6);
}

// ---------------------------------------------------------------------------
// Workspace records of the draw.

struct DrawSeg {       // one (prefix, segment)
  double sp, sq;       // sum of w_p, w_q (residual: relative to the row max;
                       // bonus: relative to the segment max)
  double ap, aq;       // sums of w_p, w_q over sure-positive tokens (residual)
  float mseg;          // bonus: raw max logit of the segment
  int last_pos;        // last sure-positive token (residual), -1 if none
  int last_p;          // last token with w_p > 0, -1 if none
  int n_unc;           // stored uncertain tokens, -1 when the list overflowed
  int bad;             // bonus: a NaN logit in the segment
  int pad;
};

struct DrawUnc {       // one uncertain token
  double wp, wq;
  int v, pad;
};

struct DrawMass {      // one (prefix, segment) after the pick's first stage
  double zr;           // residual mass (or p mass for a bonus draw)
  double zp;           // p mass (fallback when the residual has no mass)
  int last_r, last_p;
  int pad[2];
};

template <typename E>
struct DrawRows {
  const typename E::elem *p;
  const typename E::elem *q;  // nullptr for a bonus draw
};

// Rows taken from pools through index tables ([B][K][gamma+1] and
// [B][K][gamma]); null tables mean the dense layout.
struct RowIndex {
  const int32_t *p;
  const int32_t *q;
};

template <typename E>
__device__ __forceinline__ DrawRows<E> draw_rows(const typename E::elem *p, const typename E::elem *q,
                                                 const RowIndex ix, int K, int gamma, int V,
                                                 int64_t b, const DrawDesc &d) {
  const int64_t bk = b * K + d.k;
  const int64_t pr = ix.p ? (int64_t)ix.p[bk * (gamma + 1) + d.pos] : bk * (gamma + 1) + d.pos;
  DrawRows<E> r;
  r.p = p + pr * (int64_t)V;
  r.q = nullptr;
  if (d.two) {
    const int64_t qr = ix.q ? (int64_t)ix.q[bk * gamma + d.pos] : bk * gamma + d.pos;
    r.q = q + qr * (int64_t)V;
  }
  return r;
}

// Visit the logits of [lo, hi) of one or two rows with NT threads: f(v, zp, zq).
// kVec: rows start 16-byte aligned and hi - lo is a multiple of a vector.
template <typename E, bool kVec, bool kTwo, int NT, typename F>
__device__ __forceinline__ void visit_segment(const typename E::elem *rp, const typename E::elem *rq,
                                     int lo, int hi, F &&f) {
  if constexpr (kVec) {
    constexpr int P = E::kPerVec;
    const vec16 *vp = reinterpret_cast<const vec16 *>(rp);
    const vec16 *vq = reinterpret_cast<const vec16 *>(rq);
    for (int i = lo / P + (int)threadIdx.x; i < hi / P; i += NT) {
      float xp[P], xq[P];
      E::unpack(vp[i], xp);
      if constexpr (kTwo) E::unpack(vq[i], xq);
#pragma unroll
      for (int e = 0; e < P; ++e) f(i * P + e, xp[e], kTwo ? xq[e] : 0.0f);
    }
  } else {
    for (int v = lo + (int)threadIdx.x; v < hi; v += NT)
      f(v, E::at(rp, v), kTwo ? E::at(rq, v) : 0.0f);
  }
}

// One reduction of a segment's four sums and two last indices (fixed order);
// the results are valid in thread 0 only.
template <int NW>
__device__ __forceinline__ void block_reduce_seg(double &a, double &b, double &c, double &d,
                                                 int &x, int &y, double *ldsd /* 4*NW */,
                                                 int *ldsi /* 2*NW */) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a += __shfl_xor(a, off, 64);
    b += __shfl_xor(b, off, 64);
    c += __shfl_xor(c, off, 64);
    d += __shfl_xor(d, off, 64);
    x = max(x, __shfl_xor(x, off, 64));
    y = max(y, __shfl_xor(y, off, 64));
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    ldsd[4 * w] = a;
    ldsd[4 * w + 1] = b;
    ldsd[4 * w + 2] = c;
    ldsd[4 * w + 3] = d;
    ldsi[2 * w] = x;
    ldsi[2 * w + 1] = y;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll 1
    for (int i = 1; i < NW; ++i) {
      a += ldsd[4 * i];
      b += ldsd[4 * i + 1];
      c += ldsd[4 * i + 2];
      d += ldsd[4 * i + 3];
      x = max(x, ldsi[2 * i]);
      y = max(y, ldsi[2 * i + 1]);
    }
  }
  __syncthreads();
}

// Segment seg of one prefix in the draw's fp64 pass, for the decision d and
// (residual draws) the drawn row pair's statistics st.
template <typename E, bool kVec, int NT>
__device__ __forceinline__ void draw_pass_item(const typename E::elem *__restrict__ p,
                                               const typename E::elem *__restrict__ q,
                                               const RowIndex ix, int K, int gamma, int V,
                                               int nseg, float tp, float tq, const DrawDesc d,
                                               const RowStats st,
                                               DrawSeg *__restrict__ segs,
                                               DrawUnc *__restrict__ uncs, int64_t b, int seg) {
  constexpr int NW = NT / 64;
  __shared__ Exp64Table tab;
  __shared__ float ldsf[NW + 1];
  __shared__ double ldsd[4 * NW];
  __shared__ int ldsi[2 * NW + 1];
  __shared__ int n_unc;
  __shared__ DrawUnc unc[kUncCap];
  if (!d.valid) return;
  exp64_table_init(tab);
  const DrawRows<E> r = draw_rows<E>(p, q, ix, K, gamma, V, b, d);
  const double invTp = 1.0 / (double)tp, invTq = 1.0 / (double)tq;
  if (threadIdx.x == 0) n_unc = 0;
  __syncthreads();
  const int lo = seg * kDrawSeg, hi = min(V, lo + kDrawSeg);
  double sp = 0.0, sq = 0.0, ap = 0.0, aq = 0.0;
  int last_pos = -1, last_p = -1, bad = 0;
  float mseg = kNegInf;
  if (d.two) {
    const double Mp = (double)st.mp / (double)tp, Mq = (double)st.mq / (double)tq;
    const double rho = (double)st.sp / (double)st.sq;  // fp32 estimate of S_p / S_q
    const double up = rho * (1.0 + kClassMargin), dn = rho * (1.0 - kClassMargin);
    visit_segment<E, kVec, true, NT>(r.p, r.q, lo, hi, [&](int v, float zp, float zq) {
      const double wp = exp_nonpos(__builtin_fma((double)zp, invTp, -Mp), tab);
      const double wq = exp_nonpos(__builtin_fma((double)zq, invTq, -Mq), tab);
      sp += wp;
      sq += wq;
      if (wp > 0.0) last_p = v;
      if (wp > up * wq) {
        ap += wp;
        aq += wq;
        last_pos = v;
      } else if (wp > 0.0 && wp >= dn * wq) {  // rare: inside the margin
        const int i = atomicAdd(&n_unc, 1);
        if (i < kUncCap) unc[i] = DrawUnc{wp, wq, v, 0};
      }
    });
  } else {
    float m = kNegInf;
    visit_segment<E, kVec, false, NT>(r.p, r.p, lo, hi, [&](int, float zp, float) {
      m = fmaxf(m, zp);
      bad |= (zp != zp);
    });
    mseg = block_max<NW>(m, ldsf);
    bad = block_max_i<NW>(bad, ldsi);
    const double M = (double)fmaxf(mseg, kLowest) / (double)tp;
    const int excl = d.excl;  // sp: every token; ap: all but the excluded one
    visit_segment<E, kVec, false, NT>(r.p, r.p, lo, hi, [&](int v, float zp, float) {
      const double wp = exp_nonpos(__builtin_fma((double)zp, invTp, -M), tab);
      sp += wp;
      if (wp > 0.0) last_p = v;
      if (v != excl) {
        ap += wp;
        if (wp > 0.0) last_pos = v;
      }
    });
  }
  block_reduce_seg<NW>(sp, sq, ap, aq, last_pos, last_p, ldsd, ldsi);
  // uncertain tokens in token order (distinct tokens: the ranks are a permutation)
  const int64_t so = b * nseg + seg;
  const int n = n_unc;
  if (n <= kUncCap && (int)threadIdx.x < n) {
    const DrawUnc e = unc[threadIdx.x];
    int rank = 0;
    for (int i = 0; i < n; ++i) rank += (unc[i].v < e.v);
    uncs[so * kUncCap + rank] = e;
  }
  if (threadIdx.x == 0) {
    DrawSeg out{};
    out.sp = sp;
    out.sq = sq;
    out.ap = ap;
    out.aq = aq;
    out.last_pos = last_pos;
    out.last_p = last_p;
    out.mseg = mseg;
    out.bad = bad;
    out.n_unc = (n > kUncCap) ? -1 : n;
    segs[so] = out;
  }
}

// decision and drawn-row statistics from the workspace (separate launches)
__device__ __forceinline__ RowStats drawn_stats(const RowStats *stats, const DrawDesc &d, int K,
                                                int gamma, int64_t b) {
  if (d.valid && d.two) return stats[(b * K + d.k) * gamma + d.pos];
  return RowStats{0.0f, 1.0f, 0.0f, 1.0f};
}

template <typename E, bool kVec>
__global__ __launch_bounds__(kBlock) void kr_draw_pass(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q,
    const RowIndex ix, int K, int gamma, int V, int nseg, float tp, float tq,
    const RowStats *__restrict__ stats, const DrawDesc *__restrict__ desc,
    DrawSeg *__restrict__ segs, DrawUnc *__restrict__ uncs) {
  const int64_t b = blockIdx.x / nseg;
  const DrawDesc d = desc[b];
  draw_pass_item<E, kVec, kBlock>(p, q, ix, K, gamma, V, nseg, tp, tq, d,
                                  drawn_stats(stats, d, K, gamma, b), segs, uncs, b,
                                  (int)(blockIdx.x - b * nseg));
}

// Exact weights of the draw.
template <typename E>
struct DrawWeight {
  const typename E::elem *p, *q;
  double invTp, invTq, Mp, Mq, invSp, invSq;
  bool resid;  // max(0, p - q); otherwise p with token excl zeroed
  int excl;
  // weight of token v from its two logits
  __device__ __forceinline__ double from(int v, float zp, float zq, const Exp64Table &tab) const {
    const double pv = exp_nonpos(__builtin_fma((double)zp, invTp, -Mp), tab) * invSp;
    if (!resid) return v == excl ? 0.0 : pv;
    const double qv = exp_nonpos(__builtin_fma((double)zq, invTq, -Mq), tab) * invSq;
    const double dd = pv - qv;
    return dd > 0.0 ? dd : 0.0;
  }
};

// Exact row normalisers of the draw from the pass's segment sums, in segment
// order (the fix and the pick run this same code, so they agree to the bit).
// Returns false for an invalid bonus row.
template <typename E>
__device__ __forceinline__ bool draw_setup(const DrawRows<E> &rows, const DrawDesc &d,
                                           const RowStats &st, const DrawSeg *S, int nseg,
                                           float tp, float tq, DrawWeight<E> &W) {
  W.p = rows.p;
  W.q = rows.q;
  W.invTp = 1.0 / (double)tp;
  W.invTq = 1.0 / (double)tq;
  W.resid = d.two != 0;
  W.excl = d.excl;
  double Sp = 0.0, Sq = 1.0;
  if (W.resid) {
    W.Mp = (double)st.mp / (double)tp;
    W.Mq = (double)st.mq / (double)tq;
    Sq = 0.0;
    for (int s = 0; s < nseg; ++s) {
      const DrawSeg g = S[s];
      Sp += g.sp;
      Sq += g.sq;
    }
  } else {
    float mr = kNegInf;
    int bad = 0;
    for (int s = 0; s < nseg; ++s) {
      const DrawSeg g = S[s];
      mr = fmaxf(mr, g.mseg);
      bad |= g.bad;
    }
    if (bad || mr == kNegInf || mr == -kNegInf) return false;
    W.Mp = (double)mr / (double)tp;
    W.Mq = 0.0;
    for (int s = 0; s < nseg; ++s) {
      const DrawSeg g = S[s];
      const double Ms = (double)fmaxf(g.mseg, kLowest) / (double)tp;
      Sp += (g.mseg == mr) ? g.sp : g.sp * exp(Ms - W.Mp);
    }
  }
  W.invSp = 1.0 / Sp;
  W.invSq = 1.0 / Sq;
  return true;
}

// Exact residual mass of one segment (all NT threads); valid in thread 0.
template <typename E, bool kVec, int NT>
__device__ __forceinline__ void segment_mass_exact(const DrawWeight<E> &W, const DrawSeg &S, int V,
                                                   int seg, const Exp64Table &tab, double *ldsd,
                                                   int *ldsi, DrawMass &m) {
  const int lo = seg * kDrawSeg, hi = min(V, lo + kDrawSeg);
  double z = 0.0;
  int last = -1;
  visit_segment<E, kVec, true, NT>(W.p, W.q, lo, hi, [&](int v, float zp, float zq) {
    const double w = W.from(v, zp, zq, tab);
    z += w;
    if (w > 0.0) last = v;
  });
  m.zr = block_sum_d<NT / 64>(z, ldsd);
  m.last_r = block_max_i<NT / 64>(last, ldsi);
  m.zp = S.sp * W.invSp;
  m.last_p = S.last_p;
}

// (prefix, segment): exact residual mass of a segment whose uncertain list
// overflowed; every other workgroup returns at once.
template <typename E, bool kVec>
__global__ __launch_bounds__(kBlock) void kr_draw_fix(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q,
    const RowIndex ix, int K, int gamma, int V, int nseg, float tp, float tq,
    const RowStats *__restrict__ stats,
    const DrawDesc *__restrict__ desc, const DrawSeg *__restrict__ segs,
    DrawMass *__restrict__ mass) {
  __shared__ Exp64Table tab;
  __shared__ double ldsd[kWaves + 1];
  __shared__ int ldsi[kWaves + 1];
  const int64_t b = blockIdx.x / nseg;
  const int seg = (int)(blockIdx.x - b * nseg);
  const DrawDesc d = desc[b];
  const DrawSeg *S = segs + b * nseg;
  if (!d.valid || !d.two || S[seg].n_unc >= 0) return;
  exp64_table_init(tab);
  __syncthreads();
  const DrawRows<E> rows = draw_rows<E>(p, q, ix, K, gamma, V, b, d);
  DrawWeight<E> W;
  draw_setup<E>(rows, d, drawn_stats(stats, d, K, gamma, b), S, nseg, tp, tq, W);
  DrawMass m{};
  segment_mass_exact<E, kVec, kBlock>(W, S[seg], V, seg, tab, ldsd, ldsi, m);
  if (threadIdx.x == 0) mass[b * nseg + seg] = m;
}

// Exclusive prefix sum over the workgroup in thread order (fixed pattern).
template <int NW>
__device__ __forceinline__ double block_exclusive_scan(double x, double *lds /* NW */) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(inc, off, 64);
    if (lane >= off) inc += y;
  }
  if (lane == 63) lds[w] = inc;
  __syncthreads();
  double base = 0.0;
#pragma unroll 1
  for (int i = 0; i < w; ++i) base += lds[i];
  const double prev = __shfl_up(inc, 1, 64);
  __syncthreads();
  return base + (lane == 0 ? 0.0 : prev);
}

// The pick for one prefix, for the decision d and the drawn row pair's
// statistics st.  The masses of segments whose uncertain list overflowed come
// from kr_draw_fix.
template <typename E, bool kVec, int NT>
__device__ __forceinline__ void draw_pick_item(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q,
    const RowIndex ix, int K, int gamma, int V, int nseg, float tp, float tq, uint64_t seed,
    uint64_t row_base,
    const DrawDesc d, const RowStats st, const DrawSeg *__restrict__ segs,
    const DrawUnc *__restrict__ uncs, DrawMass *__restrict__ mass,
    int32_t *__restrict__ selected, int32_t *__restrict__ accept_len,
    int32_t *__restrict__ next_token, int64_t b, bool inline_fix) {
  constexpr int NW = NT / 64;
  constexpr int kRun = kDrawSeg / NT;  // tokens per thread in the scan of one segment
  __shared__ Exp64Table tab;
  __shared__ double ldsd[NW + 1];
  __shared__ int ldsi[NW + 1];
  __shared__ DrawSeg segl[kPickSegs];   // the prefix's segment records, when they fit
  __shared__ DrawMass massl[kPickSegs];
  const int tid = threadIdx.x;
  if (!d.valid) return;
  exp64_table_init(tab);
  // the serial loops below read the segment records from LDS (global memory
  // for vocabularies of more than kPickSegs segments)
  const bool staged = nseg <= kPickSegs;
  if (staged)
    for (int s = tid; s < nseg; s += NT) segl[s] = segs[b * nseg + s];
  __syncthreads();
  const DrawRows<E> rows = draw_rows<E>(p, q, ix, K, gamma, V, b, d);
  const DrawSeg *S = staged ? segl : segs + b * nseg;
  DrawMass *msg = mass + b * nseg;  // the fix kernel's masses
  DrawMass *ms = staged ? massl : msg;
  const bool residual = d.two != 0;
  DrawWeight<E> W;
  if (!draw_setup<E>(rows, d, st, S, nseg, tp, tq, W)) {
    if (tid == 0) {  // invalid bonus row (the scored rows were checked earlier)
      if (selected) selected[b] = -1;
      accept_len[b] = -1;
      next_token[b] = -1;
    }
    return;
  }

  // per-segment masses of the other segments
  for (int s = tid; s < nseg; s += NT) {
    const DrawSeg g = S[s];
    if (residual && g.n_unc < 0) {  // recomputed by the fix kernel, or just below
      if (staged && !inline_fix) ms[s] = msg[s];
      continue;
    }
    DrawMass m{};
    m.last_p = g.last_p;
    if (residual) {
      m.zp = g.sp * W.invSp;
      double z = g.ap * W.invSp - g.aq * W.invSq;
      int last = g.last_pos;
      const DrawUnc *u = uncs + (b * nseg + s) * kUncCap;
      for (int i = 0; i < g.n_unc; ++i) {
        const DrawUnc e = u[i];
        const double dd = e.wp * W.invSp - e.wq * W.invSq;
        if (dd > 0.0) {
          z += dd;
          last = max(last, e.v);
        }
      }
      m.zr = z;
      m.last_r = last;
    } else {  // p row: zp with every token, zr without the excluded one
      const double Ms = (double)fmaxf(g.mseg, kLowest) / (double)tp;
      const double scale = (g.mseg == kNegInf) ? 0.0 : exp(Ms - W.Mp);
      m.zp = g.sp * scale * W.invSp;
      m.zr = g.ap * scale * W.invSp;
      m.last_r = g.last_pos;
    }
    ms[s] = m;
  }
  __syncthreads();
  if (inline_fix && residual) {  // few prefixes: overflowed segments settled here
    for (int s = 0; s < nseg; ++s) {
      const DrawSeg g = S[s];
      if (g.n_unc >= 0) continue;
      DrawMass m{};
      segment_mass_exact<E, kVec, NT>(W, g, V, s, tab, ldsd, ldsi, m);
      if (tid == 0) ms[s] = m;
    }
    __syncthreads();
  }

  double zr = 0.0;
  for (int s = 0; s < nseg; ++s) zr += ms[s].zr;
  const bool use_r = zr > 0.0;  // a residual without mass draws from p
  W.resid = residual && use_r;
  if (!use_r) W.excl = -1;
  double Z = zr;
  if (!use_r) {
    Z = 0.0;
    for (int s = 0; s < nseg; ++s) Z += ms[s].zp;
  }
  const double t = counter_uniform(seed, row_base + (uint64_t)b, (uint64_t)d.pos,
                                   (uint64_t)d.purpose) * Z;

  double cum = 0.0;
  int s0 = -1;
  for (int s = 0; s < nseg; ++s) {
    const double w = use_r ? ms[s].zr : ms[s].zp;
    if (cum + w > t) {
      s0 = s;
      break;
    }
    cum += w;
  }
  int tok = -1;
  if (s0 >= 0) {
    for (int s = s0; s < nseg; ++s) {
      // thread tid owns tokens [a, a + kRun) of the segment, kept in registers
      const int lo = s * kDrawSeg, hi = min(V, lo + kDrawSeg);
      const int a = lo + tid * kRun;
      double w[kRun];
      if constexpr (kVec) {
        constexpr int P = E::kPerVec;
        static_assert(kRun % P == 0, "a run is whole 16-byte vectors");
        const vec16 *vp = reinterpret_cast<const vec16 *>(W.p + a);
        const vec16 *vq = reinterpret_cast<const vec16 *>(W.q + (W.resid ? a : 0));
#pragma unroll
        for (int c = 0; c < kRun / P; ++c) {
          float xp[P], xq[P];
          if (a + c * P < hi) {  // hi - lo is a multiple of P on this path
            E::unpack(vp[c], xp);
            if (W.resid) E::unpack(vq[c], xq);
          }
#pragma unroll
          for (int e = 0; e < P; ++e)
            w[c * P + e] =
                (a + c * P < hi) ? W.from(a + c * P + e, xp[e], W.resid ? xq[e] : 0.0f, tab) : 0.0;
        }
      } else {
#pragma unroll
        for (int i = 0; i < kRun; ++i) {
          const int v = a + i;
          w[i] = (v < hi) ? W.from(v, E::at(W.p, v), W.resid ? E::at(W.q, v) : 0.0f, tab) : 0.0;
        }
      }
      double loc = 0.0;
#pragma unroll
      for (int i = 0; i < kRun; ++i) loc += w[i];
      double C = cum + block_exclusive_scan<NW>(loc, ldsd);
      int found = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kRun; ++i) {
        C += w[i];
        if (found == 0x7fffffff && w[i] > 0.0 && C > t) found = a + i;
      }
      found = block_min_i<NW>(found, ldsi);
      if (found != 0x7fffffff) {
        tok = found;
        break;
      }
      cum += use_r ? ms[s].zr : ms[s].zp;
    }
  }
  if (tok < 0) {  // t at or past the total through rounding
    for (int s = 0; s < nseg; ++s) tok = max(tok, use_r ? ms[s].last_r : ms[s].last_p);
  }
  if (tid == 0) next_token[b] = tok;
}

template <typename E, bool kVec>
__global__ __launch_bounds__(kBlock) void kr_draw_pick(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q,
    const RowIndex ix, int K, int gamma, int V, int nseg, float tp, float tq, uint64_t seed,
    uint64_t row_base,
    const RowStats *__restrict__ stats, const DrawDesc *__restrict__ desc,
    const DrawSeg *__restrict__ segs, const DrawUnc *__restrict__ uncs,
    DrawMass *__restrict__ mass, int32_t *__restrict__ selected,
    int32_t *__restrict__ accept_len, int32_t *__restrict__ next_token, int inline_fix) {
  const int64_t b = blockIdx.x;
  const DrawDesc d = desc[b];
  draw_pick_item<E, kVec, kBlock>(p, q, ix, K, gamma, V, nseg, tp, tq, seed, row_base, d,
                                  drawn_stats(stats, d, K, gamma, b), segs, uncs, mass, selected,
                                  accept_len, next_token, b, inline_fix != 0);
}

}  // namespace svd
