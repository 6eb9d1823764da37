// kr_beta.hpp -- overlap mass beta = sum_v min(p_v, q_v) of every scored row
// pair, the expected acceptance of a position with a fresh draft x ~ q
// (1 - total variation; the residual of SpecDiff-2 section 2 carries the
// remaining 1 - beta).  It needs the final normalisers, so it is a second
// pass over the rows, run only when the caller asks for beta.
#pragma once

#include "svd_device.hpp"

namespace svd {

template <typename E, bool kVec>
__global__ __launch_bounds__(kBlock) void kr_beta(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q, int gamma,
    int V, float cp, float cq, const RowStats *__restrict__ stats, float *__restrict__ beta) {
  __shared__ float lds[kWaves + 1];
  const int64_t rp = blockIdx.x;
  const int64_t bk = rp / gamma;
  const int64_t j = rp - bk * gamma;
  const typename E::elem *prow = p + (bk * (gamma + 1) + j) * (int64_t)V;
  const typename E::elem *qrow = q + rp * (int64_t)V;
  const RowStats st = stats[rp];
  const bool ok = !(st.sp != st.sp) && !(st.sq != st.sq) && st.mp != kNegInf && st.mq != kNegInf;
  if (!ok) {
    if (threadIdx.x == 0) beta[rp] = __builtin_nanf("");
    return;
  }
  const float ip = 1.0f / st.sp, iq = 1.0f / st.sq;
  float acc = 0.0f;
  if constexpr (kVec) {
    constexpr int P = E::kPerVec;
    const vec16 *vp = reinterpret_cast<const vec16 *>(prow);
    const vec16 *vq = reinterpret_cast<const vec16 *>(qrow);
    for (int i = threadIdx.x; i < V / P; i += kBlock) {
      float xp[P], xq[P];
      E::unpack(__builtin_nontemporal_load(vp + i), xp);
      E::unpack(__builtin_nontemporal_load(vq + i), xq);
#pragma unroll
      for (int e = 0; e < P; ++e)
        acc += fminf(fast_exp2((xp[e] - st.mp) * cp) * ip, fast_exp2((xq[e] - st.mq) * cq) * iq);
    }
  } else {
    for (int i = threadIdx.x; i < V; i += kBlock)
      acc += fminf(fast_exp2((E::at(prow, i) - st.mp) * cp) * ip,
                   fast_exp2((E::at(qrow, i) - st.mq) * cq) * iq);
  }
  const float sum = block_sum_f<kWaves>(acc, lds);
  if (threadIdx.x == 0) beta[rp] = sum;
}

}  // namespace svd
