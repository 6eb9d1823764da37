// kr_beta.hpp -- overlap mass beta = sum_v min(p_v, q_v) of every scored row
// pair, the expected acceptance of a position with a fresh draft x ~ q
// (1 - total variation; the residual of SpecDiff-2 section 2 carries the
// remaining 1 - beta).  It needs the final normalisers, so it is a second
// pass over the rows, run only when the caller asks for beta.
#pragma once

#include "svd_device.hpp"

namespace svd {

// One workgroup per (row pair, slice of S): [sl * slice, sl * slice + slice)
// of the vocabulary (slice: whole 16-byte loads on the vector path).  With
// S == 1 the row pair's beta is written directly; otherwise part[] gets the
// slice's sum and kr_beta_combine adds the S sums in slice order.  Two
// vectors of each row are loaded per step (four loads in flight per thread),
// taken in the same order as one at a time, so a row's sum keeps its bits.
template <typename E, bool kVec>
__global__ __launch_bounds__(kBlock) void kr_beta(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q, int gamma,
    int V, float cp, float cq, const RowStats *__restrict__ stats, int S, int slice,
    float *__restrict__ beta, float *__restrict__ part) {
  __shared__ float lds[kWaves + 1];
  const int64_t rp = blockIdx.x / S;
  const int sl = (int)(blockIdx.x - rp * S);
  const int64_t bk = rp / gamma;
  const int64_t j = rp - bk * gamma;
  const typename E::elem *prow = p + (bk * (gamma + 1) + j) * (int64_t)V;
  const typename E::elem *qrow = q + rp * (int64_t)V;
  const int lo = sl * slice, hi = min(V, lo + slice);
  float *out = S == 1 ? beta + rp : part + blockIdx.x;
  const RowStats st = stats[rp];
  const bool ok = !(st.sp != st.sp) && !(st.sq != st.sq) && st.mp != kNegInf && st.mq != kNegInf;
  if (!ok) {
    if (threadIdx.x == 0) *out = __builtin_nanf("");
    return;
  }
  const float ip = 1.0f / st.sp, iq = 1.0f / st.sq;
  float acc = 0.0f;
  if constexpr (kVec) {
    constexpr int P = E::kPerVec;
    const vec16 *vp = reinterpret_cast<const vec16 *>(prow);
    const vec16 *vq = reinterpret_cast<const vec16 *>(qrow);
    auto add = [&](const vec16 &a, const vec16 &b) {
      float xp[P], xq[P];
      E::unpack(a, xp);
      E::unpack(b, xq);
#pragma unroll
      for (int e = 0; e < P; ++e)
        acc += fminf(fast_exp2((xp[e] - st.mp) * cp) * ip, fast_exp2((xq[e] - st.mq) * cq) * iq);
    };
    const int iend = hi / P;
    int i = lo / P + (int)threadIdx.x;
    for (; i + kBlock < iend; i += 2 * kBlock) {
      const vec16 a0 = __builtin_nontemporal_load(vp + i), b0 = __builtin_nontemporal_load(vq + i);
      const vec16 a1 = __builtin_nontemporal_load(vp + i + kBlock);
      const vec16 b1 = __builtin_nontemporal_load(vq + i + kBlock);
      add(a0, b0);
      add(a1, b1);
    }
    if (i < iend) add(__builtin_nontemporal_load(vp + i), __builtin_nontemporal_load(vq + i));
  } else {
    for (int i = lo + (int)threadIdx.x; i < hi; i += kBlock)
      acc += fminf(fast_exp2((E::at(prow, i) - st.mp) * cp) * ip,
                   fast_exp2((E::at(qrow, i) - st.mq) * cq) * iq);
  }
  const float sum = block_sum_f<kWaves>(acc, lds);
  if (threadIdx.x == 0) *out = sum;
}

// beta of each row pair from its S slice sums, added in slice order (a NaN
// slice, from an invalid row pair, makes the sum NaN).
__global__ __launch_bounds__(kBlock) void kr_beta_combine(int64_t rows, int S,
                                                          const float *__restrict__ part,
                                                          float *__restrict__ beta) {
  const int64_t rp = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (rp >= rows) return;
  const float *pp = part + rp * S;
  float sum = pp[0];
  for (int k = 1; k < S; ++k) sum += pp[k];
  beta[rp] = sum;
}

}  // namespace svd
