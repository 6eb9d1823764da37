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
// The drawn rows are recomputed from the logits in fp64, in three launches
// over vocabulary segments of kDrawSeg tokens:
//   kr_draw_sums  (prefix, segment): segment max and sum of exp(z/T - m_seg)
//   kr_draw_mass  (prefix, segment): exact row normalisers from all segments,
//                 then the segment's residual mass and last weighted index
//   kr_draw_pick  (prefix): find the segment holding t, then an LDS prefix
//                 sum over thread-contiguous runs locates the token.
// Every reduction has a fixed order, so the result is deterministic.
#pragma once

#include "svd_device.hpp"

namespace svd {

template <typename E>
struct DrawRows {
  const typename E::elem *p;
  const typename E::elem *q;  // nullptr for a bonus draw
};

template <typename E>
__device__ inline DrawRows<E> draw_rows(const typename E::elem *p, const typename E::elem *q,
                                        int K, int gamma, int V, int64_t b, const DrawDesc &d) {
  const int64_t bk = b * K + d.k;
  DrawRows<E> r;
  r.p = p + (bk * (gamma + 1) + d.pos) * (int64_t)V;
  r.q = (d.purpose == kResidual) ? q + (bk * gamma + d.pos) * (int64_t)V : nullptr;
  return r;
}

// max and fp64 sum of exp(z/T - m_seg) over row[lo, hi); valid in all threads
template <typename E>
__device__ inline void seg_sums(const typename E::elem *row, int lo, int hi, float T,
                                float &m_raw, double &S, float *ldsf, double *ldsd) {
  float m = kNegInf;
  for (int v = lo + (int)threadIdx.x; v < hi; v += kBlock) m = fmaxf(m, E::at(row, v));
  m = block_max(m, ldsf);
  const double Td = (double)T;
  const double M = (double)fmaxf(m, kLowest) / Td;
  const double invT = 1.0 / Td;
  double s = 0.0;
  for (int v = lo + (int)threadIdx.x; v < hi; v += kBlock)
    s += exp((double)E::at(row, v) * invT - M);  // NaN logits poison the sum
  S = block_sum_d(s, ldsd);
  m_raw = m;
}

// Row normaliser from the per-segment sums, in segment order.  The same code
// runs in kr_draw_mass and kr_draw_pick, so both see the same bits.
__device__ inline bool row_norm(const DrawSums *s, int nseg, bool use_q, float T, double &M,
                                double &S) {
  float mr = kNegInf;
  for (int i = 0; i < nseg; ++i) mr = fmaxf(mr, use_q ? s[i].mq : s[i].mp);
  const double Td = (double)T;
  M = (double)mr / Td;
  double acc = 0.0;
  for (int i = 0; i < nseg; ++i) {
    const float mi = use_q ? s[i].mq : s[i].mp;
    const double si = use_q ? s[i].sq : s[i].sp;
    acc += (mi == mr) ? si : si * exp((double)mi / Td - M);
  }
  S = acc;
  return mr != kNegInf && mr != -kNegInf && acc == acc && acc > 0.0;
}

template <typename E>
__global__ __launch_bounds__(kBlock) void kr_draw_sums(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q, int K,
    int gamma, int V, int nseg, float tp, float tq, const DrawDesc *__restrict__ desc,
    DrawSums *__restrict__ sums) {
  __shared__ float ldsf[kWaves];
  __shared__ double ldsd[kWaves];
  const int64_t b = blockIdx.x / nseg;
  const int seg = (int)(blockIdx.x - b * nseg);
  const DrawDesc d = desc[b];
  if (!d.valid) return;
  const DrawRows<E> r = draw_rows<E>(p, q, K, gamma, V, b, d);
  const int lo = seg * kDrawSeg, hi = min(V, lo + kDrawSeg);
  DrawSums out{};
  seg_sums<E>(r.p, lo, hi, tp, out.mp, out.sp, ldsf, ldsd);
  if (r.q) {
    seg_sums<E>(r.q, lo, hi, tq, out.mq, out.sq, ldsf, ldsd);
  } else {
    out.mq = kNegInf;
    out.sq = 0.0;
  }
  if (threadIdx.x == 0) sums[b * nseg + seg] = out;
}

// weight of token v in the draw
template <typename E>
struct DrawWeight {
  const typename E::elem *p, *q;
  double invTp, invTq, Mp, Mq, invSp, invSq;
  bool resid;
  __device__ inline void at(int v, double &w, double &pv) const {
    pv = exp((double)E::at(p, v) * invTp - Mp) * invSp;
    if (resid) {
      const double qv = exp((double)E::at(q, v) * invTq - Mq) * invSq;
      const double d = pv - qv;
      w = d > 0.0 ? d : 0.0;
    } else {
      w = pv;
    }
  }
};

template <typename E>
__device__ inline bool make_weight(const DrawRows<E> &r, const DrawSums *s, int nseg, float tp,
                                   float tq, DrawWeight<E> &w) {
  double Sp, Sq = 1.0;
  bool ok = row_norm(s, nseg, false, tp, w.Mp, Sp);
  w.Mq = 0.0;
  if (r.q) ok = row_norm(s, nseg, true, tq, w.Mq, Sq) && ok;
  w.p = r.p;
  w.q = r.q;
  w.invTp = 1.0 / (double)tp;
  w.invTq = 1.0 / (double)tq;
  w.invSp = 1.0 / Sp;
  w.invSq = 1.0 / Sq;
  w.resid = r.q != nullptr;
  return ok;
}

template <typename E>
__global__ __launch_bounds__(kBlock) void kr_draw_mass(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q, int K,
    int gamma, int V, int nseg, float tp, float tq, const DrawDesc *__restrict__ desc,
    const DrawSums *__restrict__ sums, DrawMass *__restrict__ mass) {
  __shared__ double ldsd[kWaves];
  __shared__ int ldsi[kWaves];
  const int64_t b = blockIdx.x / nseg;
  const int seg = (int)(blockIdx.x - b * nseg);
  const DrawDesc d = desc[b];
  if (!d.valid) return;
  const DrawRows<E> r = draw_rows<E>(p, q, K, gamma, V, b, d);
  DrawWeight<E> W;
  if (!make_weight<E>(r, sums + b * nseg, nseg, tp, tq, W)) return;  // the pick reports it
  const int lo = seg * kDrawSeg, hi = min(V, lo + kDrawSeg);
  double zr = 0.0, zp = 0.0;
  int lr = -1, lp = -1;
  for (int v = lo + (int)threadIdx.x; v < hi; v += kBlock) {
    double w, pv;
    W.at(v, w, pv);
    zr += w;
    zp += pv;
    if (w > 0.0) lr = v;
    if (pv > 0.0) lp = v;
  }
  DrawMass out{};
  out.zr = block_sum_d(zr, ldsd);
  out.zp = block_sum_d(zp, ldsd);
  out.last_r = block_max_i(lr, ldsi);
  out.last_p = block_max_i(lp, ldsi);
  if (threadIdx.x == 0) mass[b * nseg + seg] = out;
}

template <typename E>
__global__ __launch_bounds__(kBlock) void kr_draw_pick(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q, int K,
    int gamma, int V, int nseg, float tp, float tq, uint64_t seed, uint64_t row_base,
    const DrawDesc *__restrict__ desc, const DrawSums *__restrict__ sums,
    const DrawMass *__restrict__ mass, int32_t *__restrict__ selected,
    int32_t *__restrict__ accept_len, int32_t *__restrict__ next_token) {
  __shared__ double scan[kBlock];
  __shared__ int ldsi[kWaves];
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  const DrawDesc d = desc[b];
  if (!d.valid) return;
  const DrawRows<E> r = draw_rows<E>(p, q, K, gamma, V, b, d);
  DrawWeight<E> W;
  if (!make_weight<E>(r, sums + b * nseg, nseg, tp, tq, W)) {
    // only a bonus row can be invalid here: the scored rows were checked
    if (tid == 0) {
      if (selected) selected[b] = -1;
      accept_len[b] = -1;
      next_token[b] = -1;
    }
    return;
  }
  const DrawMass *ms = mass + b * nseg;
  double zr = 0.0;
  for (int s = 0; s < nseg; ++s) zr += ms[s].zr;
  const bool resid = W.resid && zr > 0.0;
  W.resid = resid;  // no residual mass: draw from p
  double Z = zr;
  if (!resid) {
    Z = 0.0;
    for (int s = 0; s < nseg; ++s) Z += ms[s].zp;
  }
  const double t = counter_uniform(seed, row_base + (uint64_t)b, (uint64_t)d.pos,
                                   (uint64_t)d.purpose) * Z;

  double cum = 0.0;
  int s0 = -1;
  for (int s = 0; s < nseg; ++s) {
    const double w = resid ? ms[s].zr : ms[s].zp;
    if (cum + w > t) {
      s0 = s;
      break;
    }
    cum += w;
  }
  int tok = -1;
  if (s0 >= 0) {
    for (int s = s0; s < nseg; ++s) {
      const int lo = s * kDrawSeg, hi = min(V, lo + kDrawSeg);
      const int chunk = (hi - lo + kBlock - 1) / kBlock;
      const int a = min(hi, lo + tid * chunk), e = min(hi, a + chunk);
      double loc = 0.0;
      for (int v = a; v < e; ++v) {
        double w, pv;
        W.at(v, w, pv);
        loc += w;
      }
      scan[tid] = loc;
      __syncthreads();
      if (tid == 0) {  // exclusive prefix sum in thread order
        double run = 0.0;
        for (int i = 0; i < kBlock; ++i) {
          const double x = scan[i];
          scan[i] = run;
          run += x;
        }
      }
      __syncthreads();
      double C = cum + scan[tid];
      int found = 0x7fffffff;
      for (int v = a; v < e; ++v) {
        double w, pv;
        W.at(v, w, pv);
        C += w;
        if (w > 0.0 && C > t) {
          found = v;
          break;
        }
      }
      found = block_min_i(found, ldsi);
      if (found != 0x7fffffff) {
        tok = found;
        break;
      }
      cum += resid ? ms[s].zr : ms[s].zp;
    }
  }
  if (tok < 0) {  // t at or past the total through rounding
    for (int s = 0; s < nseg; ++s) tok = max(tok, resid ? ms[s].last_r : ms[s].last_p);
  }
  if (tid == 0) next_token[b] = tok;
}

}  // namespace svd
