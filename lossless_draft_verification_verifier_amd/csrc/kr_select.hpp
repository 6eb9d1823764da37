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

// Ragged, EOS-aware windows (DiffuSpec section 3, "Accepted prefix length";
// section 4.3): draft k's usable positions are j < m_k = mlen[b*K+k] (the
// window gamma_b[b], cut after the draft's first EOS; -1 for a window outside
// [1, gamma]).  Scores and acceptance stop there; a fully accepted window that
// ends in EOS commits without a draw (next_token = -2), and the bonus comes
// from p row gamma_b[b].
struct Window {
  const int32_t *mlen;     // null: every window is gamma, no EOS
  const int32_t *gamma_b;  // null: gamma
  int eos;                 // -1: none
  int first_only;          // K == 1, positions streamed only up to the first rejection:
                           // no scores, alpha read only up to it
};

// Run by the 64 lanes of one wave (lane = threadIdx.x & 63); every lane gets
// the decision.  Lane 0 writes selected / accept_len (and -1 next_token for an
// invalid prefix), lane k writes scores[k].  p_index (nullable): the verifier
// rows come from a pool of np rows, and a bonus row outside it makes the
// prefix invalid.
__device__ __forceinline__ DrawDesc select_prefix(const float *__restrict__ alpha_ws,
                                                  const int32_t *__restrict__ drafts, bool greedy,
                                                  const int32_t *__restrict__ p_index, int64_t np,
                                                  const Window win, int K, int gamma,
                                                  uint64_t seed, uint64_t row_base, int64_t b,
                                                  int32_t *__restrict__ selected,
                                                  int32_t *__restrict__ accept_len,
                                                  int32_t *__restrict__ next_token,
                                                  float *__restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int n = win.gamma_b ? win.gamma_b[b] : gamma;  // the window (bonus row n)
  auto usable = [&](int k) { return win.mlen ? win.mlen[(int64_t)b * K + k] : gamma; };
  double S = -1.0;
  bool bad = false;
  if (lane < K && !win.first_only) {
    const int64_t base = ((int64_t)b * K + lane) * gamma;
    const int m = usable(lane);
    bad |= m < 1;
    double prod = 1.0;
    S = 0.0;
    for (int j = 0; j < m; ++j) {
      const float aj = alpha_ws[base + j];
      bad |= (aj != aj);
      prod *= (double)aj;
      S += prod;
    }
    if (scores) scores[b * K + lane] = (float)S;
  }
  bool invalid = __any(bad) || (win.first_only && usable(0) < 1);

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

  const int m = invalid ? 0 : usable(bk);
  int L = m;
  if (!invalid) {
    const int64_t base = ((int64_t)b * K + bk) * gamma;
    const uint64_t row = row_base + (uint64_t)b;
    for (int j0 = 0; j0 < m; j0 += 64) {
      const int j = j0 + lane;
      bool rej = false;
      if (j < m)
        rej = !(counter_uniform(seed, row, (uint64_t)j, kAccept) < (double)alpha_ws[base + j]);
      const uint64_t mask = __ballot(rej);
      if (mask) {
        L = j0 + __ffsll((unsigned long long)mask) - 1;
        break;
      }
    }
    // streamed up to the first rejection only: its alpha is the one that can be NaN
    if (win.first_only && L < m) invalid = alpha_ws[base + L] != alpha_ws[base + L];
  }

  // an accepted window that ends in EOS commits without a draw
  const bool eos_end = !invalid && L == m && win.eos >= 0 &&
                       drafts[((int64_t)b * K + bk) * gamma + m - 1] == win.eos;
  if (!invalid && !eos_end && L == m && p_index) {
    const int32_t pi = p_index[((int64_t)b * K + bk) * (gamma + 1) + n];
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
      if (eos_end) next_token[b] = -2;
    }
  }
  if (invalid || eos_end) return DrawDesc{0, 0, 0, 0, 0, -1};
  if (L == m) return DrawDesc{bk, n, (int)kBonus, 1, 0, -1};
  if (greedy)
    return DrawDesc{bk, L, (int)kResidual, 1, 0, drafts[((int64_t)b * K + bk) * gamma + L]};
  return DrawDesc{bk, L, (int)kResidual, 1, 1, -1};
}

__global__ __launch_bounds__(64) void kr_select(
    const float *__restrict__ alpha_ws, const int32_t *__restrict__ drafts, int greedy,
    const int32_t *__restrict__ p_index, int64_t np, const Window win, int K, int gamma,
    uint64_t seed, uint64_t row_base, int32_t *__restrict__ selected,
    int32_t *__restrict__ accept_len, int32_t *__restrict__ next_token,
    float *__restrict__ scores, DrawDesc *__restrict__ desc) {
  const DrawDesc d = select_prefix(alpha_ws, drafts, greedy != 0, p_index, np, win, K, gamma,
                                   seed, row_base, blockIdx.x, selected, accept_len, next_token,
                                   scores);
  if (threadIdx.x == 0) desc[blockIdx.x] = d;
}

// Usable length of every draft: its window, cut after its first EOS; -1 for a
// window outside [1, gamma].
__global__ __launch_bounds__(kBlock) void kr_window(const int32_t *__restrict__ drafts,
                                                    const int32_t *__restrict__ gamma_b, int eos,
                                                    int64_t BK, int K, int gamma,
                                                    int32_t *__restrict__ mlen) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;  // b * K + k
  if (i >= BK) return;
  const int n = gamma_b ? gamma_b[i / K] : gamma;
  int m = (n < 1 || n > gamma) ? -1 : n;
  for (int j = 0; j < m && eos >= 0; ++j)
    if (drafts[i * gamma + j] == eos) {
      m = j + 1;
      break;
    }
  mlen[i] = m;
}

// One draft per prefix, positions [j0, j0 + jn) just streamed: a draft whose
// first rejection falls there stops being streamed.
__global__ __launch_bounds__(kBlock) void kr_advance(const float *__restrict__ alpha_ws,
                                                     const int32_t *__restrict__ mlen, int64_t B,
                                                     int gamma, int j0, int jn, uint64_t seed,
                                                     uint64_t row_base,
                                                     uint32_t *__restrict__ alive) {
  const int64_t b = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (b >= B || !alive[b]) return;
  const int m = mlen[b];
  for (int j = j0; j < j0 + jn && j < m; ++j)
    if (!(counter_uniform(seed, row_base + (uint64_t)b, (uint64_t)j, kAccept) <
          (double)alpha_ws[b * gamma + j])) {
      alive[b] = 0u;
      return;
    }
}

}  // namespace svd
