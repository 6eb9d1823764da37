// kr_rowstats.hpp -- row statistics and acceptance of every scored row pair.
//
// One workgroup per (prefix b, draft k, position j < gamma).  It streams the
// verifier row p(.|s, x_<j) and the drafter row q(.|s, x_<j) once, keeping an
// online (max, sum) of exp2((z - max) * log2(e) / T) per thread, merges the
// threads, and turns the two rows' statistics into
//   alpha = min(1, p(x_j) / q(x_j))
// (SpecDiff-2 section 2: accept at once whenever q <= p; Figure 2's
// position-wise acceptance).  alpha is formed from log2-probabilities so it
// stays defined when both probabilities are tiny.  Invalid rows or tokens give
// alpha = NaN, which the selection epilogue turns into -1 outputs.
//
// Memory: 16-byte coalesced nontemporal loads when every row starts 16-byte
// aligned (the row length in bytes is a multiple of 16), otherwise one element
// per load.
#pragma once

#include "svd_device.hpp"

namespace svd {

// Launch shape of the standalone streaming kernel (from a sweep of threads
// per workgroup and loads in flight): 1024 threads, two 16-byte loads in
// flight per thread and row.
constexpr int kRowBlock = 1024;
constexpr int kRowUnroll = 2;

// Streaming loads are nontemporal: every logit byte is read once.
__device__ __forceinline__ vec16 stream_load(const vec16 *p) {
  return __builtin_nontemporal_load(p);
}

// Fold one vector of n logits into a thread's (max, sum) state.
template <int N>
__device__ __forceinline__ void ms_fold(float &m, float &s, const float *x, float c) {
  float vm = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) vm = fmaxf(vm, x[i]);
  const float mn = fmaxf(m, vm);  // fmaxf drops NaN: a NaN logit shows up in the sum
  s *= (mn == m) ? 1.0f : fast_exp2((m - mn) * c);
  m = mn;
  const float mo = fmaxf(m, kLowest);  // keeps (-inf) - (-inf) out of the exponent
#pragma unroll
  for (int i = 0; i < N; ++i) s += fast_exp2((x[i] - mo) * c);
}

// (max, sum) of one row over NT threads with U loads in flight per thread;
// the result is valid in thread 0.
template <typename E, bool kVec, int NT, int U>
__device__ __forceinline__ void row_ms(const typename E::elem *row, int V, float c, float &m_out,
                              float &s_out, float *lds) {
  float m[U], s[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    m[u] = kNegInf;
    s[u] = 0.0f;
  }
  const int tid = threadIdx.x;
  if constexpr (kVec) {
    constexpr int P = E::kPerVec;
    const vec16 *vrow = reinterpret_cast<const vec16 *>(row);
    const int nvec = V / P;  // V * sizeof(elem) is a multiple of 16 on this path
    int i = tid;
    for (; i + (U - 1) * NT < nvec; i += U * NT) {
      vec16 w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) w[u] = stream_load(vrow + i + u * NT);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x[P];
        E::unpack(w[u], x);
        ms_fold<P>(m[u], s[u], x, c);
      }
    }
    for (; i < nvec; i += NT) {
      vec16 w = stream_load(vrow + i);
      float x[P];
      E::unpack(w, x);
      ms_fold<P>(m[0], s[0], x, c);
    }
  } else {
    int i = tid;
    for (; i + (U - 1) * NT < V; i += U * NT) {
      float x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = E::at(row, i + u * NT);
#pragma unroll
      for (int u = 0; u < U; ++u) ms_fold<1>(m[u], s[u], &x[u], c);
    }
    for (; i < V; i += NT) {
      float x = E::at(row, i);
      ms_fold<1>(m[0], s[0], &x, c);
    }
  }
#pragma unroll
  for (int u = 1; u < U; ++u) ms_merge(m[0], s[0], m[u], s[u], c);
  block_ms<NT / 64>(m[0], s[0], c, lds);
  m_out = m[0];
  s_out = s[0];
}

// alpha of one scored position from its two rows' statistics (raw max m and
// sum s of exp2((z - m) * c)) and the drafted token's logits; NaN when a row
// is invalid.  kGreedy: alpha = p(x), the q row is ignored.
template <bool kGreedy>
__device__ __forceinline__ float acceptance(float zpx, float mp, float sp, float cp, float zqx,
                                            float mq, float sq, float cq) {
  const bool rows_ok = !(sp != sp) && !(sq != sq) && mp != kNegInf && mq != kNegInf;
  if (!rows_ok) return __builtin_nanf("");
  // log2 p(x) (and log2 q(x)); accept outright when q(x) <= p(x)
  const float lp = (zpx - mp) * cp - log2f(sp);
  if constexpr (kGreedy) {
    return fminf(exp2f(lp), 1.0f);
  } else {
    const float lq = (zqx - mq) * cq - log2f(sq);
    return (lq <= lp) ? 1.0f : exp2f(lp - lq);
  }
}

// One scored row pair: statistics of both rows and alpha, written by thread 0.
// kGreedy: greedy acceptance (SpecDiff-2 section 5.2 and appendix B.4), which
// compares the uniform with the verifier probability of the drafted token, so
// alpha = p(x) and the drafter row is not read (its statistics are left as
// {0, 1}).
template <typename E, bool kVec, int NT, int U, bool kGreedy = false>
__device__ __forceinline__ void rowstats_item(const typename E::elem *__restrict__ p,
                                     const typename E::elem *__restrict__ q,
                                     const int32_t *__restrict__ drafts, int gamma, int V,
                                     float cp, float cq, int64_t rp, RowStats *__restrict__ stats,
                                     float *__restrict__ alpha_ws, float *__restrict__ alpha_out) {
  __shared__ float lds[2 * (NT / 64)];
  const int64_t bk = rp / gamma;  // rp = (b * K + k) * gamma + j
  const int64_t j = rp - bk * gamma;
  const typename E::elem *prow = p + (bk * (gamma + 1) + j) * (int64_t)V;
  const typename E::elem *qrow = kGreedy ? nullptr : q + rp * (int64_t)V;

  float mp, sp, mq = 0.0f, sq = 1.0f;
  row_ms<E, kVec, NT, U>(prow, V, cp, mp, sp, lds);
  if constexpr (!kGreedy) row_ms<E, kVec, NT, U>(qrow, V, cq, mq, sq, lds);

  if (threadIdx.x == 0) {
    const int32_t x = drafts[rp];
    float a = __builtin_nanf("");
    if (x >= 0 && x < V)
      a = acceptance<kGreedy>(E::at(prow, x), mp, sp, cp, kGreedy ? 0.0f : E::at(qrow, x), mq,
                              sq, cq);
    stats[rp] = RowStats{mp, sp, mq, sq};
    alpha_ws[rp] = a;
    if (alpha_out) alpha_out[rp] = a;
  }
}

// Workgroup w takes position j = j0 + w % jn of draft (b, k) = w / jn (the
// whole batch: j0 = 0, jn = gamma).  Ragged or EOS-aware windows: mlen[b*K+k]
// is the draft's usable length and later positions are skipped; positions
// streamed in chunks: alive[b*K+k] == 0 skips a draft already rejected.  A
// skipped position's alpha output is NaN.
// Two 1024-thread workgroups per CU (8 waves per SIMD) need at most 64 VGPRs.
// Rows of fewer than kShortRowBytes take NT = kShortRowBlock threads (eight
// workgroups per CU), so that a thread still has several loads per row.
constexpr int kShortRowBlock = 256;
constexpr int64_t kShortRowBytes = 128 * 1024;

template <typename E, bool kVec, bool kGreedy, int NT = kRowBlock>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8))) void kr_rowstats(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q,
    const int32_t *__restrict__ drafts, int gamma, int V, float cp, float cq,
    RowStats *__restrict__ stats, float *__restrict__ alpha_ws, float *__restrict__ alpha_out,
    const int32_t *__restrict__ mlen, const uint32_t *__restrict__ alive, int j0, int jn) {
  const int64_t bk = blockIdx.x / jn;
  const int j = j0 + (int)(blockIdx.x - bk * jn);
  if (j >= gamma) return;
  const int64_t rp = bk * gamma + j;
  if ((mlen && j >= mlen[bk]) || (alive && !alive[bk])) {
    if (alpha_out && threadIdx.x == 0) alpha_out[rp] = __builtin_nanf("");
    return;
  }
  rowstats_item<E, kVec, NT, kRowUnroll, kGreedy>(p, q, drafts, gamma, V, cp, cq, rp, stats,
                                                  alpha_ws, alpha_out);
}

// ---------------------------------------------------------------------------
// Split rows.  A launch with few row pairs (a single sequence, or the later
// chunks of an early exit) cannot fill the GPU with one workgroup per pair, so
// each pair's vocabulary is cut into S slices of whole 16-byte vectors, one
// 256-thread workgroup per slice writes a partial (max, sum) record of both
// rows, and kr_rowstats_combine merges the S records of a pair in slice order
// and forms alpha.

constexpr int kSplitBlock = 256;

struct PartStats {  // one (row pair, slice)
  float mp, sp, mq, sq;
};

// Workgroup w: slice w % S of launch row r = w / S, i.e. position j0 + r % jn
// of draft r / jn; skipping as in kr_rowstats.
template <typename E, bool kVec, bool kGreedy>
__global__ __launch_bounds__(kSplitBlock) void kr_rowstats_split(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q, int gamma,
    int V, float cp, float cq, int S, int slice, const int32_t *__restrict__ mlen,
    const uint32_t *__restrict__ alive, int j0, int jn, PartStats *__restrict__ part) {
  __shared__ float lds[2 * (kSplitBlock / 64)];
  const int64_t r = blockIdx.x / S;
  const int sl = (int)(blockIdx.x - r * S);
  const int64_t bk = r / jn;
  const int j = j0 + (int)(r - bk * jn);
  if (j >= gamma || (mlen && j >= mlen[bk]) || (alive && !alive[bk])) return;
  const int lo = sl * slice, hi = min(V, lo + slice);  // slice: whole vectors
  const typename E::elem *prow = p + (bk * (gamma + 1) + j) * (int64_t)V + lo;
  float mp, sp, mq = 0.0f, sq = 1.0f;
  row_ms<E, kVec, kSplitBlock, kRowUnroll>(prow, hi - lo, cp, mp, sp, lds);
  if constexpr (!kGreedy) {
    const typename E::elem *qrow = q + (bk * gamma + j) * (int64_t)V + lo;
    row_ms<E, kVec, kSplitBlock, kRowUnroll>(qrow, hi - lo, cq, mq, sq, lds);
  }
  if (threadIdx.x == 0) part[blockIdx.x] = PartStats{mp, sp, mq, sq};
}

// One launch row r merged by one wave: lane sl holds slice sl's record (lane
// sl + 64k folds slices past 64 in first), a butterfly merges the lanes in a
// fixed pattern, and lane 0 forms alpha.
template <typename E, bool kGreedy>
__device__ __forceinline__ void combine_row(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q,
    const int32_t *__restrict__ drafts, int64_t rows, int gamma, int V, float cp, float cq, int S,
    const int32_t *__restrict__ mlen, const uint32_t *__restrict__ alive, int j0, int jn,
    const PartStats *__restrict__ part, RowStats *__restrict__ stats,
    float *__restrict__ alpha_ws, float *__restrict__ alpha_out, int64_t r, int lane) {
  if (r >= rows) return;  // whole waves
  const int64_t bk = r / jn;
  const int j = j0 + (int)(r - bk * jn);
  if (j >= gamma) return;
  const int64_t rp = bk * gamma + j;
  if ((mlen && j >= mlen[bk]) || (alive && !alive[bk])) {
    if (alpha_out && lane == 0) alpha_out[rp] = __builtin_nanf("");
    return;
  }
  PartStats a{kNegInf, 0.0f, kNegInf, 0.0f};
  for (int sl = lane; sl < S; sl += 64) {
    const PartStats b = part[r * S + sl];
    ms_merge(a.mp, a.sp, b.mp, b.sp, cp);
    if constexpr (!kGreedy) ms_merge(a.mq, a.sq, b.mq, b.sq, cq);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    ms_merge(a.mp, a.sp, __shfl_xor(a.mp, off, 64), __shfl_xor(a.sp, off, 64), cp);
    if constexpr (!kGreedy)
      ms_merge(a.mq, a.sq, __shfl_xor(a.mq, off, 64), __shfl_xor(a.sq, off, 64), cq);
  }
  if (lane != 0) return;
  if constexpr (kGreedy) {
    a.mq = 0.0f;
    a.sq = 1.0f;
  }
  const int32_t x = drafts[rp];
  float al = __builtin_nanf("");
  if (x >= 0 && x < V)
    al = acceptance<kGreedy>(E::at(p + (bk * (gamma + 1) + j) * (int64_t)V, x), a.mp, a.sp, cp,
                             kGreedy ? 0.0f : E::at(q + rp * (int64_t)V, x), a.mq, a.sq, cq);
  stats[rp] = RowStats{a.mp, a.sp, a.mq, a.sq};
  alpha_ws[rp] = al;
  if (alpha_out) alpha_out[rp] = al;
}

// One wave per launch row.
template <typename E, bool kGreedy>
__global__ __launch_bounds__(kBlock) void kr_rowstats_combine(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q,
    const int32_t *__restrict__ drafts, int64_t rows, int gamma, int V, float cp, float cq, int S,
    const int32_t *__restrict__ mlen, const uint32_t *__restrict__ alive, int j0, int jn,
    const PartStats *__restrict__ part, RowStats *__restrict__ stats,
    float *__restrict__ alpha_ws, float *__restrict__ alpha_out) {
  const int64_t r = ((int64_t)blockIdx.x * kBlock + threadIdx.x) >> 6;
  combine_row<E, kGreedy>(p, q, drafts, rows, gamma, V, cp, cq, S, mlen, alive, j0, jn, part,
                          stats, alpha_ws, alpha_out, r, threadIdx.x & 63);
}

}  // namespace svd

namespace svd {

// ---------------------------------------------------------------------------
// Early exit over a live list.  One draft per prefix is streamed in chunks of
// J positions; the prefixes not yet rejected form a list (live, its length in
// a device counter) that the merge of each chunk rebuilds for the next.  A
// chunk's launch has a fixed grid of kLiveGrid workgroups and cuts each of
// its n * J rows into as many slices as fill that grid, so the later chunks,
// with few prefixes left, still spread over every CU.  The slicing depends
// only on n, so a row's statistics do not depend on which prefixes are live.
constexpr int kLiveGrid = 1024;

struct LivePlan {
  int S;      // slices per row
  int slice;  // elements per slice (whole loads)
};

// units: loads per row (V / elements per load); Smax: most slices per row
__device__ __forceinline__ LivePlan live_plan(int64_t rows, int units, int unit, int Smax) {
  int64_t s = rows > 0 ? kLiveGrid / rows : 1;
  s = s < 1 ? 1 : (s > Smax ? Smax : s);
  const int su = (int)((units + s - 1) / s);  // loads per slice
  return LivePlan{(units + su - 1) / su, su * unit};
}

// Workgroup w: slice w % S of row r = w / S, i.e. position j0 + r % J of the
// prefix live[r / J]; positions past the prefix's usable length are skipped.
template <typename E, bool kVec, bool kGreedy>
__global__ __launch_bounds__(kSplitBlock) void kr_rowstats_live(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q, int gamma,
    int V, float cp, float cq, int units, int unit, int Smax, const int32_t *__restrict__ mlen,
    const int32_t *__restrict__ live, const uint32_t *__restrict__ count, int j0, int J,
    PartStats *__restrict__ part) {
  __shared__ float lds[2 * (kSplitBlock / 64)];
  const int64_t rows = (int64_t)*count * J;
  const LivePlan L = live_plan(rows, units, unit, Smax);
  const int64_t item = blockIdx.x;
  if (item >= rows * L.S) return;
  const int64_t r = item / L.S;
  const int sl = (int)(item - r * L.S);
  const int64_t w = r / J;
  const int j = j0 + (int)(r - w * J);
  const int64_t b = live[w];
  if (j >= gamma || j >= mlen[b]) return;
  const int lo = sl * L.slice, hi = min(V, lo + L.slice);
  const typename E::elem *prow = p + (b * (gamma + 1) + j) * (int64_t)V + lo;
  float mp, sp, mq = 0.0f, sq = 1.0f;
  row_ms<E, kVec, kSplitBlock, kRowUnroll>(prow, hi - lo, cp, mp, sp, lds);
  if constexpr (!kGreedy) {
    const typename E::elem *qrow = q + (b * gamma + j) * (int64_t)V + lo;
    row_ms<E, kVec, kSplitBlock, kRowUnroll>(qrow, hi - lo, cq, mq, sq, lds);
  }
  if (threadIdx.x == 0) part[item] = PartStats{mp, sp, mq, sq};
}

}  // namespace svd
