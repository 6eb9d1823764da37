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
// The selection has already settled the drawn rows and their statistics
// (DrawDesc).  The rows are recomputed from the logits in fp64, in two
// launches:
//
// kr_draw_pass (prefix, vocabulary segment of kDrawSeg tokens), one fp64 pass:
//   residual draw: with the exact row maxima from the row-statistics kernel,
//     w_p = exp(z_p/T_p - M_p) and w_q likewise; the segment sums of w_p and
//     w_q give the exact normalisers S_p, S_q.  Whether p_v > q_v, i.e.
//     w_p > (S_p/S_q) w_q, is decided against the fp32 ratio from the
//     row-statistics kernel with a relative margin kClassMargin far above its
//     error, without branches: sure-positive tokens add w_p and w_q to two
//     more segment sums, so sum_v max(0, p_v - q_v) over them is
//     (sum w_p)/S_p - (sum w_q)/S_q.  The rare tokens inside the margin are
//     settled once S_p and S_q are known.  At equal temperatures the ratio
//     p_v / q_v of a token depends only on the logit difference
//     d = z_p - z_q (it is exp(d/T + M_q - M_p) S_q / S_p up to rounding), and
//     bf16 logits put hundreds of tokens on each difference, so a margin
//     token's difference is its class: tokens with d = 0 go to two more sums,
//     the others are collected in LDS and, when more than kUncCap, merged
//     class by class; a class has one sign, and a token whose own sign could
//     differ from it is within 1e-12 of p_v = q_v, where its weight is below
//     rounding.  At most kUncCap entries (single tokens or classes) are kept
//     per segment.
//   p-row draw (bonus, or greedy rejection): segment max, then the sums of
//     exp(z/T - m_seg) with and without the excluded token.
// kr_draw_pick (prefix, kPickBlock threads): exact normalisers and segment
//   masses (a segment whose uncertain list overflowed is recomputed here, all
//   threads on one segment), the segment that holds t, then each thread takes
//   kRun consecutive tokens of that segment into registers and a workgroup
//   prefix sum over the threads' totals locates the token.  The rare fallback
//   (t at or past the total) scans segments from the end for the last token
//   with weight.
// Every reduction has a fixed order and the uncertain tokens are summed in
// token order, so the result is deterministic.
#pragma once

#include "svd_device.hpp"

namespace svd {

#ifndef SVD_UNC_CAP
#define SVD_UNC_CAP 32
#endif
constexpr int kUncCap = SVD_UNC_CAP;   // uncertain tokens kept per segment
#ifndef SVD_PICK_BLOCK
#define SVD_PICK_BLOCK 256
#endif
constexpr int kPickBlock = SVD_PICK_BLOCK;  // threads of a pick workgroup
constexpr int kUncList = 512;          // margin tokens a pass workgroup collects
constexpr int kPickSegs = 256;         // segment records the pick stages in LDS
constexpr int kPickUncSegs = 32;       // segments whose uncertain lists the pick stages
constexpr double kClassMargin = 2e-4;  // relative margin of the p > q test

// ---------------------------------------------------------------------------
// exp(x) in fp64 for x <= 0 (a few ulp above 0 is fine; x must not be NaN):
// x = n ln2/64 + r with |r| <= ln2/128, n rounded to nearest by the 1.5 * 2^52
// shifter in one fma (its low word is n); r by a Cody-Waite split of ln2/64
// (n ln2_hi is exact for |n| < 2^17); exp(r) by its degree-5 Taylor
// polynomial (the next term is below 4e-17); 2^(n mod 64 / 64) from a 64-entry
// table; then ldexp by n div 64.

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

template <int NT>
__device__ __forceinline__ void exp64_table_init(Exp64Table &tab) {
  for (int i = threadIdx.x; i < 64; i += NT) tab.t[i] = kExp2Frac64[i];
}

__device__ __forceinline__ double exp_nonpos(double x, const Exp64Table &tab) {
  constexpr double kShift = 0x1.8p52;
  x = fmax(x, -760.0);  // exp(-760) is 0 in double; also maps -inf
  const double y = __builtin_fma(x, 92.33248261689366, kShift);  // 64 / ln 2
  const double n = y - kShift;
  const int ni = (int)(uint32_t)__builtin_bit_cast(uint64_t, y);
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
  double sp, sq;       // sums of w_p, w_q (residual: relative to the row max;
                       // p-row draw: relative to the segment max)
  double ap, aq;       // residual: sums of w_p, w_q over sure-positive tokens;
                       // p-row draw: ap = sum of w_p without the excluded token
  double ep, eq;       // residual: sums of w_p, w_q over margin tokens of equal logits
  float mseg;          // p-row draw: raw max logit of the segment
  int n_unc;           // stored uncertain tokens, -1 when the list overflowed
  int bad;             // p-row draw: a NaN logit in the segment
  int pad;
};

struct DrawUnc {       // one margin token, or one class of them (sums of its weights)
  double wp, wq;
  int v, pad;          // the token (the class's first token)
};

struct DrawMass {      // one (prefix, segment) in the pick
  double zr;           // residual mass (or p mass without the excluded token)
  double zp;           // p mass (fallback when the residual has no mass)
};

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

// Sums of N doubles over the workgroup in a fixed order; valid in thread 0.
template <int NW, int N>
__device__ __forceinline__ void block_sums(double (&x)[N], double *lds /* N*NW */) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += __shfl_xor(x[i], off, 64);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int i = 0; i < N; ++i) lds[N * w + i] = x[i];
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll 1
    for (int k = 1; k < NW; ++k)
#pragma unroll
      for (int i = 0; i < N; ++i) x[i] += lds[N * k + i];
  }
  __syncthreads();
}

// Segment seg of one prefix in the draw's fp64 pass.
template <typename E, bool kVec, int NT>
__device__ __forceinline__ void draw_pass_item(const typename E::elem *__restrict__ p,
                                               const typename E::elem *__restrict__ q, int V,
                                               int nseg, float tp, float tq, const DrawDesc d,
                                               DrawSeg *__restrict__ segs,
                                               DrawUnc *__restrict__ uncs, int64_t b, int seg) {
  constexpr int NW = NT / 64;
  __shared__ Exp64Table tab;
  __shared__ float ldsf[NW + 1];
  __shared__ double ldsd[6 * NW];
  __shared__ int ldsi[NW + 1];
  __shared__ int n_unc;
  __shared__ DrawUnc unc[kUncList];
  __shared__ double ukey[kUncList];  // the tokens' logit differences
  __shared__ int uord[kUncList];
  if (!d.valid) return;
  exp64_table_init<NT>(tab);
  const typename E::elem *rp = p + d.prow * (int64_t)V;
  const double invTp = 1.0 / (double)tp, invTq = 1.0 / (double)tq;
  if (threadIdx.x == 0) n_unc = 0;
  __syncthreads();
  const int lo = seg * kDrawSeg, hi = min(V, lo + kDrawSeg);
  double acc[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};  // sp, sq, ap, aq, ep, eq
  int bad = 0;
  float mseg = kNegInf;
  if (d.two) {
    const typename E::elem *rq = q + d.qrow * (int64_t)V;
    const double Mp = (double)d.st.mp / (double)tp, Mq = (double)d.st.mq / (double)tq;
    const double rho = (double)d.st.sp / (double)d.st.sq;  // fp32 estimate of S_p / S_q
    const double up = rho * (1.0 + kClassMargin), dn = rho * (1.0 - kClassMargin);
    const bool same_t = tp == tq;
    double sp = 0.0, sq = 0.0, ap = 0.0, aq = 0.0, ep = 0.0, eq = 0.0;
    // one vector of tokens at a time; the margin tokens of the vector are
    // settled after it, behind one branch
    constexpr int P = kVec ? E::kPerVec : 1;
    for (int i = lo / P + (int)threadIdx.x; i < (hi + P - 1) / P; i += NT) {
      float xp[P], xq[P];
      if constexpr (kVec) {
        E::unpack(reinterpret_cast<const vec16 *>(rp)[i], xp);
        E::unpack(reinterpret_cast<const vec16 *>(rq)[i], xq);
      } else {
        xp[0] = E::at(rp, i);
        xq[0] = E::at(rq, i);
      }
      double wp[P], wq[P];
      uint32_t margin = 0;
#pragma unroll
      for (int e = 0; e < P; ++e) {
        wp[e] = exp_nonpos(__builtin_fma((double)xp[e], invTp, -Mp), tab);
        wq[e] = exp_nonpos(__builtin_fma((double)xq[e], invTq, -Mq), tab);
        sp += wp[e];
        sq += wq[e];
        const bool pos = wp[e] > up * wq[e];
        const double f = pos ? 1.0 : 0.0;
        ap = __builtin_fma(f, wp[e], ap);
        aq = __builtin_fma(f, wq[e], aq);
        margin |= (uint32_t)(!pos && wp[e] > dn * wq[e]) << e;
      }
      if (margin) {  // rare
#pragma unroll
        for (int e = 0; e < P; ++e) {
          if (!((margin >> e) & 1u)) continue;
          if (same_t && xp[e] == xq[e]) {
            ep += wp[e];
            eq += wq[e];
          } else {
            const int k = atomicAdd(&n_unc, 1);
            if (k < kUncList) {
              unc[k] = DrawUnc{wp[e], wq[e], i * P + e, 0};
              ukey[k] = (double)xp[e] - (double)xq[e];
            }
          }
        }
      }
    }
    acc[0] = sp;
    acc[1] = sq;
    acc[2] = ap;
    acc[3] = aq;
    acc[4] = ep;
    acc[5] = eq;
  } else {
    float m = kNegInf;
    visit_segment<E, kVec, false, NT>(rp, rp, lo, hi, [&](int, float zp, float) {
      m = fmaxf(m, zp);
      bad |= (zp != zp);
    });
    mseg = block_max<NW>(m, ldsf);
    bad = block_max_i<NW>(bad, ldsi);
    const double M = (double)fmaxf(mseg, kLowest) / (double)tp;
    const int excl = d.excl;  // sp: every token; ap: all but the excluded one
    double sp = 0.0, ap = 0.0;
    visit_segment<E, kVec, false, NT>(rp, rp, lo, hi, [&](int v, float zp, float) {
      const double wp = exp_nonpos(__builtin_fma((double)zp, invTp, -M), tab);
      sp += wp;
      ap = __builtin_fma(v != excl ? 1.0 : 0.0, wp, ap);
    });
    acc[0] = sp;
    acc[2] = ap;
  }
  block_sums<NW, 6>(acc, ldsd);
  const int64_t so = b * nseg + seg;
  const int n = n_unc;
  int nout = -1;  // entries written; -1: the list overflowed
  if (n <= kUncCap) {
    // margin tokens in token order (distinct tokens: the ranks are a permutation)
    if ((int)threadIdx.x < n) {
      const DrawUnc e = unc[threadIdx.x];
      int rank = 0;
      for (int i = 0; i < n; ++i) rank += (unc[i].v < e.v);
      uncs[so * kUncCap + rank] = e;
    }
    nout = n;
  } else if (n <= kUncList && d.two && tp == tq) {
    // merge by class: order by (difference, token), then each class's first
    // entry sums its class in that order
    for (int i = threadIdx.x; i < n; i += NT) {
      const double ki = ukey[i];
      const int vi = unc[i].v;
      int r = 0;
      for (int j = 0; j < n; ++j) r += (ukey[j] < ki) || (ukey[j] == ki && unc[j].v < vi);
      uord[r] = i;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < n; r += NT) {
      const int i = uord[r];
      if (r > 0 && ukey[uord[r - 1]] == ukey[i]) continue;  // not the first of its class
      int g = 0;
      for (int c = 1; c <= r; ++c) g += ukey[uord[c]] != ukey[uord[c - 1]];
      if (g >= kUncCap) continue;
      double swp = 0.0, swq = 0.0;
      for (int c = r; c < n && ukey[uord[c]] == ukey[i]; ++c) {
        swp += unc[uord[c]].wp;
        swq += unc[uord[c]].wq;
      }
      uncs[so * kUncCap + g] = DrawUnc{swp, swq, unc[i].v, 0};
    }
    int ng = 1;
    for (int c = 1; c < n; ++c) ng += ukey[uord[c]] != ukey[uord[c - 1]];
    nout = ng <= kUncCap ? ng : -1;
  }
  if (threadIdx.x == 0) {
    DrawSeg out{};
    out.sp = acc[0];
    out.sq = acc[1];
    out.ap = acc[2];
    out.aq = acc[3];
    out.ep = acc[4];
    out.eq = acc[5];
    out.mseg = mseg;
    out.bad = bad;
    out.n_unc = nout;
    segs[so] = out;
  }
}

template <typename E, bool kVec>
__global__ __launch_bounds__(kBlock) void kr_draw_pass(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q, int V,
    int nseg, float tp, float tq, const DrawDesc *__restrict__ desc,
    DrawSeg *__restrict__ segs, DrawUnc *__restrict__ uncs) {
  const int64_t b = blockIdx.x / nseg;
  draw_pass_item<E, kVec, kBlock>(p, q, V, nseg, tp, tq, desc[b], segs, uncs, b,
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
// order.  Returns false for an invalid bonus row.
template <typename E>
__device__ __forceinline__ bool draw_setup(const typename E::elem *rp,
                                           const typename E::elem *rq, const DrawDesc &d,
                                           const DrawSeg *S, int nseg, float tp, float tq,
                                           DrawWeight<E> &W) {
  W.p = rp;
  W.q = rq;
  W.invTp = 1.0 / (double)tp;
  W.invTq = 1.0 / (double)tq;
  W.resid = d.two != 0;
  W.excl = d.excl;
  double Sp = 0.0, Sq = 1.0;
  if (W.resid) {
    W.Mp = (double)d.st.mp / (double)tp;
    W.Mq = (double)d.st.mq / (double)tq;
    Sq = 0.0;
    for (int s = 0; s < nseg; ++s) {
      Sp += S[s].sp;
      Sq += S[s].sq;
    }
  } else {
    float mr = kNegInf;
    int bad = 0;
    for (int s = 0; s < nseg; ++s) {
      mr = fmaxf(mr, S[s].mseg);
      bad |= S[s].bad;
    }
    if (bad || mr == kNegInf || mr == -kNegInf) return false;
    W.Mp = (double)mr / (double)tp;
    W.Mq = 0.0;
    for (int s = 0; s < nseg; ++s) {
      const double Ms = (double)fmaxf(S[s].mseg, kLowest) / (double)tp;
      Sp += (S[s].mseg == mr) ? S[s].sp : S[s].sp * exp(Ms - W.Mp);
    }
  }
  W.invSp = 1.0 / Sp;
  W.invSq = 1.0 / Sq;
  return true;
}

// The weights of the kRun consecutive tokens from a of a segment ending at hi.
template <typename E, bool kVec, int kRun>
__device__ __forceinline__ void run_weights(const DrawWeight<E> &W, int a, int hi,
                                            const Exp64Table &tab, double (&w)[kRun]) {
  if constexpr (kVec) {
    constexpr int P = E::kPerVec;
    static_assert(kRun % P == 0, "a run is whole 16-byte vectors");
    const vec16 *vp = reinterpret_cast<const vec16 *>(W.p + a);
    const vec16 *vq = reinterpret_cast<const vec16 *>(W.q + (W.resid ? a : 0));
#pragma unroll
    for (int c = 0; c < kRun / P; ++c) {
      float xp[P], xq[P];
      const bool in = a + c * P < hi;  // hi - lo is a multiple of P on this path
      if (in) {
        E::unpack(vp[c], xp);
        if (W.resid) E::unpack(vq[c], xq);
      }
#pragma unroll
      for (int e = 0; e < P; ++e)
        w[c * P + e] = in ? W.from(a + c * P + e, xp[e], W.resid ? xq[e] : 0.0f, tab) : 0.0;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      const int v = a + i;
      w[i] = (v < hi) ? W.from(v, E::at(W.p, v), W.resid ? E::at(W.q, v) : 0.0f, tab) : 0.0;
    }
  }
}

// Exact residual mass of one segment (all NT threads); valid in thread 0.
template <typename E, bool kVec, int NT>
__device__ __forceinline__ double segment_mass_exact(const DrawWeight<E> &W, int V, int seg,
                                                     const Exp64Table &tab, double *ldsd) {
  const int lo = seg * kDrawSeg, hi = min(V, lo + kDrawSeg);
  double z = 0.0;
  visit_segment<E, kVec, true, NT>(W.p, W.q, lo, hi, [&](int v, float zp, float zq) {
    z += W.from(v, zp, zq, tab);
  });
  return block_sum_d<NT / 64>(z, ldsd);
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

// The pick: one workgroup of kPickBlock threads per prefix.  mass is global
// scratch for the segment masses of vocabularies with more than kPickSegs
// segments.
template <typename E, bool kVec>
__global__ __launch_bounds__(kPickBlock) void kr_draw_pick(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q, int V,
    int nseg, float tp, float tq, uint64_t seed, uint64_t row_base,
    const DrawDesc *__restrict__ desc, const DrawSeg *__restrict__ segs,
    const DrawUnc *__restrict__ uncs, DrawMass *__restrict__ mass,
    int32_t *__restrict__ selected, int32_t *__restrict__ accept_len,
    int32_t *__restrict__ next_token) {
  constexpr int NT = kPickBlock, NW = NT / 64;
  constexpr int kRun = kDrawSeg / NT;  // tokens per thread in the scan of one segment
  __shared__ Exp64Table tab;
  __shared__ double ldsd[NW + 1];
  __shared__ int ldsi[NW + 1];
  __shared__ DrawSeg segl[kPickSegs];  // the prefix's records, when they fit
  __shared__ DrawMass massl[kPickSegs];
  __shared__ DrawUnc uncl[kPickUncSegs * kUncCap];
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  const DrawDesc d = desc[b];
  if (!d.valid) return;
  exp64_table_init<NT>(tab);
  const bool staged = nseg <= kPickSegs;
  const bool unc_staged = nseg <= kPickUncSegs;
  if (staged)
    for (int s = tid; s < nseg; s += NT) segl[s] = segs[b * nseg + s];
  if (unc_staged && d.two)  // every slot: the lists' lengths are not known yet
    for (int i = tid; i < nseg * kUncCap; i += NT) uncl[i] = uncs[b * nseg * kUncCap + i];
  __syncthreads();
  const DrawSeg *S = staged ? segl : segs + b * nseg;
  const DrawUnc *U = unc_staged ? uncl : uncs + b * nseg * kUncCap;
  DrawMass *ms = staged ? massl : mass + b * nseg;
  const typename E::elem *rp = p + d.prow * (int64_t)V;
  const typename E::elem *rq = d.two ? q + d.qrow * (int64_t)V : nullptr;
  const bool residual = d.two != 0;
  DrawWeight<E> W;
  if (!draw_setup<E>(rp, rq, d, S, nseg, tp, tq, W)) {
    if (tid == 0) {  // invalid bonus row (the scored rows were checked earlier)
      if (selected) selected[b] = -1;
      accept_len[b] = -1;
      next_token[b] = -1;
    }
    return;
  }

  // per-segment masses (the exactly recomputed residual segments just below)
  for (int s = tid; s < nseg; s += NT) {
    const DrawSeg g = S[s];
    DrawMass m{};
    if (residual) {
      m.zp = g.sp * W.invSp;
      if (g.n_unc >= 0) {
        double z = g.ap * W.invSp - g.aq * W.invSq;
        const double ze = g.ep * W.invSp - g.eq * W.invSq;  // the class of equal logits
        if (ze > 0.0) z += ze;
        const DrawUnc *u = U + (int64_t)s * kUncCap;
        for (int i = 0; i < g.n_unc; ++i) {
          const DrawUnc e = u[i];
          const double dd = e.wp * W.invSp - e.wq * W.invSq;
          if (dd > 0.0) z += dd;
        }
        m.zr = z;
      }
    } else {  // p row: zp with every token, zr without the excluded one
      const double Ms = (double)fmaxf(g.mseg, kLowest) / (double)tp;
      const double scale = (g.mseg == kNegInf) ? 0.0 : exp(Ms - W.Mp);
      m.zp = g.sp * scale * W.invSp;
      m.zr = g.ap * scale * W.invSp;
    }
    ms[s] = m;
  }
  __syncthreads();
  if (residual) {  // segments whose list overflowed: exact, all threads
    for (int s = 0; s < nseg; ++s) {
      if (S[s].n_unc >= 0) continue;
      const double z = segment_mass_exact<E, kVec, NT>(W, V, s, tab, ldsd);
      if (tid == 0) ms[s].zr = z;
      __syncthreads();
    }
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
      const int hi = min(V, (s + 1) * kDrawSeg);
      const int a = s * kDrawSeg + tid * kRun;
      double w[kRun];
      run_weights<E, kVec, kRun>(W, a, hi, tab, w);
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
  // t at or past the total through rounding: the last token with weight
  for (int s = nseg - 1; s >= 0 && tok < 0; --s) {
    const int hi = min(V, (s + 1) * kDrawSeg);
    const int a = s * kDrawSeg + tid * kRun;
    double w[kRun];
    run_weights<E, kVec, kRun>(W, a, hi, tab, w);
    int last = -1;
#pragma unroll
    for (int i = 0; i < kRun; ++i)
      if (w[i] > 0.0) last = a + i;
    tok = block_max_i<NW>(last, ldsi);
  }
  if (tid == 0) next_token[b] = tok;
}

}  // namespace svd
