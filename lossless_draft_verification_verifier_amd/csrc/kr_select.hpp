// kr_select.hpp -- streak scores, self-selection and the first rejection.
//
// One wave per prefix.  Lane k accumulates the expected accepted streak
//   S_k = sum_{j<gamma} prod_{i<=j} alpha_{k,i}
// in fp64 (SpecDiff-2 section 3: acceptance gains become longer accepted
// streaks; the score of section 5.2's self-selection).  The kept draft is the
// argmax, the lowest k on an exact tie.  Its positions are then tested left to
// right, u_j < alpha_j with u_j the counter-hash uniform of (seed, row, j,
// accept), and the accepted length L is the first failing j, or gamma
// (SpecDiff-2 section 2; DiffuSpec section 3).  The row pair of the draw is
// recorded for the sampler: position L of the kept draft for a residual
// draw, or its bonus row gamma.  Under greedy acceptance the rejection draw
// reads only the verifier row, with the rejected token zeroed (SpecDiff-2
// appendix B.4).
#pragma once

#include "svd_device.hpp"

namespace svd {

// Run by the 64 lanes of one wave (lane = threadIdx.x & 63); every lane gets
// the decision.  Lane 0 writes selected / accept_len (and -1 next_token for an
// invalid prefix), lane k writes scores[k].  p_index (nullable): the verifier
// rows come from a pool of np rows, and a bonus row outside it makes the
// prefix invalid.
__device__ __forceinline__ DrawDesc select_prefix(const float *__restrict__ alpha_ws,
                                                  const int32_t *__restrict__ drafts, bool greedy,
                                                  const int32_t *__restrict__ p_index, int64_t np,
                                                  int K, int gamma, uint64_t seed,
                                                  uint64_t row_base, int64_t b,
                                                  int32_t *__restrict__ selected,
                                                  int32_t *__restrict__ accept_len,
                                                  int32_t *__restrict__ next_token,
                                                  float *__restrict__ scores) {
  const int lane = threadIdx.x & 63;
  double S = -1.0;
  bool bad = false;
  if (lane < K) {
    const int64_t base = ((int64_t)b * K + lane) * gamma;
    double prod = 1.0;
    S = 0.0;
    for (int j = 0; j < gamma; ++j) {
      const float aj = alpha_ws[base + j];
      bad |= (aj != aj);
      prod *= (double)aj;
      S += prod;
    }
    if (scores) scores[b * K + lane] = (float)S;
  }
  bool invalid = __any(bad);

  // argmax over lanes, the lower index on an exact tie (a total order, so
  // every lane of the butterfly ends with the same winner)
  double bs = S;
  int bk = lane;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const double os = __shfl_xor(bs, off, 64);
    const int ok = __shfl_xor(bk, off, 64);
    if (os > bs || (os == bs && ok < bk)) {
      bs = os;
      bk = ok;
    }
  }

  int L = gamma;
  if (!invalid) {
    const int64_t base = ((int64_t)b * K + bk) * gamma;
    const uint64_t row = row_base + (uint64_t)b;
    for (int j0 = 0; j0 < gamma; j0 += 64) {
      const int j = j0 + lane;
      bool rej = false;
      if (j < gamma)
        rej = !(counter_uniform(seed, row, (uint64_t)j, kAccept) < (double)alpha_ws[base + j]);
      const uint64_t m = __ballot(rej);
      if (m) {
        L = j0 + __ffsll((unsigned long long)m) - 1;
        break;
      }
    }
  }

  if (!invalid && L == gamma && p_index) {
    const int32_t pi = p_index[((int64_t)b * K + bk) * (gamma + 1) + gamma];
    invalid = pi < 0 || pi >= np;
  }

  if (lane == 0) {
    if (invalid) {
      if (selected) selected[b] = -1;
      accept_len[b] = -1;
      next_token[b] = -1;
    } else {
      if (selected) selected[b] = bk;
      accept_len[b] = L;
    }
  }
  if (invalid) return DrawDesc{0, 0, 0, 0, 0, -1};
  if (L == gamma) return DrawDesc{bk, L, (int)kBonus, 1, 0, -1};
  if (greedy)
    return DrawDesc{bk, L, (int)kResidual, 1, 0, drafts[((int64_t)b * K + bk) * gamma + L]};
  return DrawDesc{bk, L, (int)kResidual, 1, 1, -1};
}

__global__ __launch_bounds__(64) void kr_select(
    const float *__restrict__ alpha_ws, const int32_t *__restrict__ drafts, int greedy,
    const int32_t *__restrict__ p_index, int64_t np, int K, int gamma, uint64_t seed,
    uint64_t row_base, int32_t *__restrict__ selected, int32_t *__restrict__ accept_len,
    int32_t *__restrict__ next_token, float *__restrict__ scores, DrawDesc *__restrict__ desc) {
  const DrawDesc d = select_prefix(alpha_ws, drafts, greedy != 0, p_index, np, K, gamma, seed,
                                   row_base, blockIdx.x, selected, accept_len, next_token,
                                   scores);
  if (threadIdx.x == 0) desc[blockIdx.x] = d;
}

}  // namespace svd
