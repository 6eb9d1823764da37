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

#include "kr_rows.hpp"  // PoolStat, alpha_row; kr_rowstats.hpp

namespace svd {

struct DrawDesc {      // one prefix: what the draw reads, settled by the selection
  int64_t prow;        // the drawn p row: row index into the p logits (or the p pool)
  int64_t qrow;        // residual draws: the q row, likewise; 0 otherwise
  RowStats st;         // statistics of the drawn row pair (when known)
  int pos;             // accepted length L (rejection) or the window (bonus)
  int purpose;         // kResidual or kBonus: the uniform's purpose
  int valid;           // 0: prefix invalid or committed without a draw
  int two;             // 1: residual max(0, p - q) of the row pair; 0: p row alone
  int excl;            // p-row draw: a token of weight zero (the rejected one), or -1
  int known;           // 1: st.mp is the drawn p row's max (a scored row); 0: bonus row
};

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
// invalid prefix), lane k writes scores[k].  p_index / q_index (nullable): the
// rows come from pools, p of np rows, and a bonus row outside it makes the
// prefix invalid.  The returned record names the rows the draw reads and,
// for a residual draw, their statistics; the loads that settle it are issued
// together with those of the acceptance test.
constexpr int kSelChunk = 16;  // alpha loads in flight per lane in the scores

// Everything the selection reads and writes.
struct SelectArgs {
  const float *alpha_ws;
  const RowStats *stats;
  const int32_t *drafts;
  int greedy;
  const int32_t *p_index, *q_index;  // nullable: shared-row pools
  int64_t np;
  Window win;
  int K, gamma;
  uint64_t seed, row_base;
  int32_t *selected, *accept_len, *next_token;
  float *scores;
};

__device__ __forceinline__ DrawDesc select_prefix(const SelectArgs &A, int64_t b) {
  const float *__restrict__ alpha_ws = A.alpha_ws;
  const RowStats *__restrict__ stats = A.stats;
  const int32_t *__restrict__ drafts = A.drafts;
  const bool greedy = A.greedy != 0;
  const int32_t *__restrict__ p_index = A.p_index;
  const int32_t *__restrict__ q_index = A.q_index;
  const int64_t np = A.np;
  const Window win = A.win;
  const int K = A.K, gamma = A.gamma;
  const uint64_t seed = A.seed, row_base = A.row_base;
  int32_t *__restrict__ selected = A.selected;
  int32_t *__restrict__ accept_len = A.accept_len;
  int32_t *__restrict__ next_token = A.next_token;
  float *__restrict__ scores = A.scores;
  const int lane = threadIdx.x & 63;
  const int n = win.gamma_b ? win.gamma_b[b] : gamma;  // the window (bonus row n)
  auto usable = [&](int k) { return win.mlen ? win.mlen[(int64_t)b * K + k] : gamma; };
  // one draft and no scores asked for: its alpha is read once, by the
  // acceptance test below (which then also finds a NaN), saving a round trip
  const bool lean = K == 1 && !scores && gamma <= 64 && !win.first_only;
  double S = -1.0;
  bool bad = false;
  if (lane < K && !win.first_only && !lean) {
    const int64_t base = ((int64_t)b * K + lane) * gamma;
    const int m = usable(lane);
    bad |= m < 1;
    double prod = 1.0;
    S = 0.0;
    for (int j0 = 0; j0 < m; j0 += kSelChunk) {
      float a[kSelChunk];
#pragma unroll
      for (int i = 0; i < kSelChunk; ++i) a[i] = (j0 + i < m) ? alpha_ws[base + j0 + i] : 1.0f;
#pragma unroll
      for (int i = 0; i < kSelChunk; ++i) {
        if (j0 + i < m) {
          bad |= (a[i] != a[i]);
          prod *= (double)a[i];
          S += prod;
        }
      }
    }
    if (scores) scores[b * K + lane] = (float)S;
  }
  bool invalid = __any(bad) || ((win.first_only || lean) && usable(0) < 1);

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
  const int64_t row_k = (int64_t)b * K + bk;  // the kept draft's rows
  const int64_t base = row_k * gamma;
  int L = m;
  RowStats st{0.0f, 1.0f, 0.0f, 1.0f};
  int xL = -1;
  int64_t prow = 0, qrow = 0;
  if (!invalid) {
    const uint64_t row = row_base + (uint64_t)b;
    for (int j0 = 0; j0 < m; j0 += 64) {
      const int j = j0 + lane;
      bool rej = false;
      float aj = 0.0f;
      RowStats sj{0.0f, 1.0f, 0.0f, 1.0f};
      int xj = -1, pj = 0, qj = 0;
      if (j < m) {
        aj = alpha_ws[base + j];
        sj = stats[base + j];
        if (greedy) xj = drafts[base + j];
        if (p_index) pj = p_index[row_k * (gamma + 1) + j];
        if (q_index && !greedy) qj = q_index[base + j];
        rej = !(counter_uniform(seed, row, (uint64_t)j, kAccept) < (double)aj);
      }
      if (lean && __any(aj != aj)) {  // the whole window is this one chunk
        invalid = true;
        break;
      }
      const uint64_t mask = __ballot(rej);
      if (mask) {
        const int src = __ffsll((unsigned long long)mask) - 1;
        L = j0 + src;
        st = RowStats{__shfl(sj.mp, src, 64), __shfl(sj.sp, src, 64), __shfl(sj.mq, src, 64),
                      __shfl(sj.sq, src, 64)};
        xL = __shfl(xj, src, 64);
        prow = p_index ? (int64_t)__shfl(pj, src, 64) : row_k * (gamma + 1) + L;
        qrow = q_index ? (int64_t)__shfl(qj, src, 64) : base + L;
        // streamed up to the first rejection only: its alpha is the one that can be NaN
        const float aL = __shfl(aj, src, 64);
        if (win.first_only) invalid = aL != aL;
        break;
      }
    }
  }

  // an accepted window that ends in EOS commits without a draw
  const bool eos_end = !invalid && L == m && win.eos >= 0 && drafts[base + m - 1] == win.eos;
  if (!invalid && !eos_end && L == m) {
    if (p_index) {
      const int32_t pi = p_index[row_k * (gamma + 1) + n];
      invalid = pi < 0 || pi >= np;
      prow = pi;
    } else {
      prow = row_k * (gamma + 1) + n;
    }
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
  DrawDesc d{};
  d.excl = -1;
  if (invalid || eos_end) return d;
  d.valid = 1;
  d.prow = prow;
  if (L == m) {
    d.pos = n;
    d.purpose = (int)kBonus;
    return d;
  }
  d.pos = L;
  d.purpose = (int)kResidual;
  d.st = st;
  d.known = 1;
  if (greedy) {
    d.excl = xL;
    return d;
  }
  d.two = 1;
  d.qrow = qrow;
  return d;
}

__global__ __launch_bounds__(64) void kr_select(const SelectArgs sel,
                                                 DrawDesc *__restrict__ desc) {
  const DrawDesc d = select_prefix(sel, blockIdx.x);
  if (threadIdx.x == 0) desc[blockIdx.x] = d;
}

// A batch of few scored rows per prefix (K * gamma <= kFuseRows) streamed as
// split rows in one launch: one workgroup per prefix merges its rows' slice
// records, a wave per row, then its wave 0 selects, so the selection takes no
// launch of its own.
constexpr int kFuseRows = 16;

template <typename E, bool kGreedy>
__global__ __launch_bounds__(64 * kFuseRows) void kr_combine_select(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q, int V,
    float cp, float cq, int S, const PartStats *__restrict__ part, RowStats *stats,
    float *alpha_ws, float *__restrict__ alpha_out, const SelectArgs sel,
    DrawDesc *__restrict__ desc) {
  // sel.stats and sel.alpha_ws are stats and alpha_ws, read back after the barrier
  const int64_t b = blockIdx.x;
  const int64_t kg = (int64_t)sel.K * sel.gamma;  // this prefix's rows
  const int64_t rows = (int64_t)gridDim.x * kg;
  combine_row<E, kGreedy>(p, q, sel.drafts, rows, sel.gamma, V, cp, cq, S, sel.win.mlen, nullptr,
                          0, sel.gamma, part, stats, alpha_ws, alpha_out,
                          b * kg + (threadIdx.x >> 6), threadIdx.x & 63);
  __syncthreads();  // the rows' alpha and statistics, visible to wave 0
  if (threadIdx.x < 64) {
    const DrawDesc d = select_prefix(sel, b);
    if (threadIdx.x == 0) desc[b] = d;
  }
}

// Shared rows with at most kAlphaSelectMax scored positions per prefix: one
// workgroup per prefix forms the alpha of its positions (a thread each, as
// kr_alpha_rows), and after the barrier wave 0 selects, so the selection
// needs no launch of its own.
constexpr int kAlphaSelectMax = 1024;

template <typename E, bool kGreedy>
__global__ __launch_bounds__(kAlphaSelectMax) void kr_alpha_select(
    const typename E::elem *__restrict__ p_pool, const typename E::elem *__restrict__ q_pool,
    int V, int64_t nq, float cp, float cq, const PoolStat *__restrict__ pstat, RowStats *stats,
    float *alpha_ws, float *__restrict__ alpha_out, const SelectArgs sel,
    DrawDesc *__restrict__ desc) {
  // sel.stats and sel.alpha_ws are stats and alpha_ws, read back after the barrier
  const int64_t b = blockIdx.x;
  const int kg = sel.K * sel.gamma;
  for (int t = threadIdx.x; t < kg; t += blockDim.x)
    alpha_row<E, kGreedy>(p_pool, q_pool, sel.p_index, sel.q_index, sel.drafts, sel.gamma, V,
                          sel.np, nq, cp, cq, pstat, stats, alpha_ws, alpha_out, b * kg + t);
  __syncthreads();  // the positions' alpha and statistics, visible to wave 0
  if (threadIdx.x < 64) {
    const DrawDesc d = select_prefix(sel, b);
    if (threadIdx.x == 0) desc[b] = d;
  }
}

// Usable length of every draft: its window, cut after its first EOS; -1 for a
// window outside [1, gamma].  Early exit over a live list (counts non-null,
// one draft per prefix): the first chunk's list holds every prefix, and the
// ncounts chunk counters start at {BK, 0, 0, ...}; the grid covers
// max(BK, ncounts) threads.
__global__ __launch_bounds__(kBlock) void kr_window(const int32_t *__restrict__ drafts,
                                                    const int32_t *__restrict__ gamma_b, int eos,
                                                    int64_t BK, int K, int gamma,
                                                    int32_t *__restrict__ mlen,
                                                    int32_t *__restrict__ live,
                                                    uint32_t *__restrict__ counts, int ncounts) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;  // b * K + k
  if (counts && i < ncounts) counts[i] = i == 0 ? (uint32_t)BK : 0u;
  if (i >= BK) return;
  if (counts) live[i] = (int32_t)i;
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

// Early exit over a live list: the merge of chunk [j0, j0 + J), one wave per
// live prefix (lanes over the slices of each row, as in combine_row; part
// null: the chunk streamed whole rows and alpha is written), then the
// chunk's acceptance tests in order.  A prefix with every test passed and
// positions left joins the next chunk's list; one that leaves the stream
// marks the alpha of its later positions NaN (not streamed).  The next list's
// order follows the atomic counter, which changes no result: each row is
// merged in slice order.
template <typename E, bool kGreedy>
__global__ __launch_bounds__(kBlock) void kr_combine_advance(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q,
    const int32_t *__restrict__ drafts, int gamma, int V, float cp, float cq, int units, int unit,
    int Smax, const int32_t *__restrict__ mlen, const int32_t *__restrict__ live,
    const uint32_t *__restrict__ count, int j0, int J, const PartStats *__restrict__ part,
    RowStats *__restrict__ stats, float *__restrict__ alpha_ws, float *__restrict__ alpha_out,
    uint64_t seed, uint64_t row_base, int32_t *__restrict__ live_next,
    uint32_t *__restrict__ count_next) {
  const int64_t n = *count;
  const int64_t w = ((int64_t)blockIdx.x * kBlock + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (w >= n) return;  // whole waves
  const LivePlan L = live_plan(n * J, units, unit, Smax);
  const int64_t b = live[w];
  const int m = mlen[b];
  bool rejected = false;
  for (int jj = 0; jj < J; ++jj) {
    const int j = j0 + jj;
    if (j >= gamma) break;
    const int64_t rp = b * gamma + j;
    if (j >= m) {
      if (alpha_out && lane == 0) alpha_out[rp] = __builtin_nanf("");
      continue;
    }
    if (!part) {  // whole rows: alpha is written already
      if (!rejected)
        rejected = !(counter_uniform(seed, row_base + (uint64_t)b, (uint64_t)j, kAccept) <
                     (double)alpha_ws[rp]);
      continue;
    }
    const int64_t r = w * J + jj;
    PartStats a{kNegInf, 0.0f, kNegInf, 0.0f};
    for (int sl = lane; sl < L.S; sl += 64) {
      const PartStats c = part[r * L.S + sl];
      ms_merge(a.mp, a.sp, c.mp, c.sp, cp);
      if constexpr (!kGreedy) ms_merge(a.mq, a.sq, c.mq, c.sq, cq);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      ms_merge(a.mp, a.sp, __shfl_xor(a.mp, off, 64), __shfl_xor(a.sp, off, 64), cp);
      if constexpr (!kGreedy)
        ms_merge(a.mq, a.sq, __shfl_xor(a.mq, off, 64), __shfl_xor(a.sq, off, 64), cq);
    }
    if constexpr (kGreedy) {
      a.mq = 0.0f;
      a.sq = 1.0f;
    }
    const int32_t x = drafts[rp];
    float al = __builtin_nanf("");
    if (x >= 0 && x < V)
      al = acceptance<kGreedy>(E::at(p + (b * (gamma + 1) + j) * (int64_t)V, x), a.mp, a.sp, cp,
                               kGreedy ? 0.0f : E::at(q + rp * (int64_t)V, x), a.mq, a.sq, cq);
    if (lane == 0) {
      stats[rp] = RowStats{a.mp, a.sp, a.mq, a.sq};
      alpha_ws[rp] = al;
      if (alpha_out) alpha_out[rp] = al;
    }
    if (!rejected)
      rejected = !(counter_uniform(seed, row_base + (uint64_t)b, (uint64_t)j, kAccept) <
                   (double)al);
  }
  const int jn = j0 + J;  // the next chunk's first position
  if (!rejected && jn < m && jn < gamma) {
    if (lane == 0) live_next[atomicAdd(count_next, 1u)] = (int32_t)b;
  } else if (alpha_out) {
    for (int j = jn + lane; j < gamma; j += 64) alpha_out[b * gamma + j] = __builtin_nanf("");
  }
}

}  // namespace svd
