// kr_rows.hpp -- scored positions whose rows come from shared pools.
//
// The K drafts of one diffusion pass are sampled from one set of drafter
// marginals, so they can share their q rows (SpecDiff-2 section 5.2); drafts
// with a common prefix share verifier rows, as in a flattened draft tree
// (SpecDiff-2 appendix B.8), and every draft of a prefix shares p row 0.  The
// caller passes a pool of verifier rows and one of drafter rows, and index
// tables p_index[B][K][gamma+1], q_index[B][K][gamma] into them.  Statistics
// are computed once per pool row that a scored position reads, so a shared row
// is streamed once:
//   kr_mark_rows:  flag every pool row read by a scored position;
//   kr_pool_stats: (max, sum) of every flagged row, one workgroup per row;
//   kr_alpha_rows: alpha of every scored position from its rows' statistics and
//                  the drafted token's two logits, plus the per-position
//                  statistics record the draw reads.
// An index outside its pool makes alpha NaN, so its prefix is reported invalid.
#pragma once

#include "kr_rowstats.hpp"

namespace svd {

struct PoolStat {  // one pool row
  float m, s;      // raw max logit, sum of exp2((z - m) * c)
};

__global__ __launch_bounds__(kBlock) void kr_fill_u32(uint32_t *__restrict__ dst, int64_t n,
                                                      uint32_t value) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) dst[i] = value;
}

// Pools of at most this many rows are flagged by one workgroup in LDS.
constexpr int kMarkLdsRows = 32768;

// flags[0, nrows) in one launch: one workgroup clears a byte per row in LDS,
// flags the rows read (as kr_mark_rows), then writes every flag out, each
// thread its own rows
__global__ __launch_bounds__(1024) void kr_mark_rows_one(const int32_t *__restrict__ p_index,
                                                         const int32_t *__restrict__ q_index,
                                                         int64_t n, int gamma, int64_t np,
                                                         int64_t nq, int64_t nrows,
                                                         uint32_t *__restrict__ flags) {
  __shared__ uint8_t f[kMarkLdsRows];
  const int tid = threadIdx.x;
  for (int64_t r = tid; r < nrows; r += 1024) f[r] = 0;
  __syncthreads();
  for (int64_t i = tid; i < n; i += 1024) {  // (b, k, j < gamma)
    const int64_t bk = i / gamma, j = i - bk * gamma;
    const int32_t pi = p_index[bk * (gamma + 1) + j];
    if (pi >= 0 && pi < np) f[pi] = 1;
    if (q_index) {
      const int32_t qi = q_index[i];
      if (qi >= 0 && qi < nq) f[np + qi] = 1;
    }
  }
  __syncthreads();
  for (int64_t r = tid; r < nrows; r += 1024) flags[r] = f[r];
}

// flags[0, np) for p rows, flags[np, np + nq) for q rows
__global__ __launch_bounds__(kBlock) void kr_mark_rows(const int32_t *__restrict__ p_index,
                                                       const int32_t *__restrict__ q_index,
                                                       int64_t n, int gamma, int64_t np,
                                                       int64_t nq, uint32_t *__restrict__ flags) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;  // (b, k, j < gamma)
  if (i >= n) return;
  const int64_t bk = i / gamma, j = i - bk * gamma;
  const int32_t pi = p_index[bk * (gamma + 1) + j];
  if (pi >= 0 && pi < np) flags[pi] = 1u;
  if (q_index) {
    const int32_t qi = q_index[i];
    if (qi >= 0 && qi < nq) flags[np + qi] = 1u;
  }
}

// NT threads per row: kRowBlock, or kShortRowBlock for rows of fewer than
// kShortRowBytes, as for kr_rowstats (the same reduction, so identity
// indices reproduce the dense statistics bit for bit)
template <typename E, bool kVec, int NT = kRowBlock>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8))) void kr_pool_stats(
    const typename E::elem *__restrict__ p_pool, const typename E::elem *__restrict__ q_pool,
    int64_t np, int V, float cp, float cq, const uint32_t *__restrict__ flags,
    PoolStat *__restrict__ pstat) {
  __shared__ float lds[2 * (NT / 64)];
  const int64_t r = blockIdx.x;  // p rows first, then q rows
  if (!flags[r]) return;
  const bool is_p = r < np;
  const typename E::elem *row = is_p ? p_pool + r * (int64_t)V : q_pool + (r - np) * (int64_t)V;
  float m, s;
  row_ms<E, kVec, NT, kRowUnroll>(row, V, is_p ? cp : cq, m, s, lds);
  if (threadIdx.x == 0) pstat[r] = PoolStat{m, s};
}

// alpha and the statistics record of scored position i = (b, k, j < gamma)
template <typename E, bool kGreedy>
__device__ __forceinline__ void alpha_row(
    const typename E::elem *__restrict__ p_pool, const typename E::elem *__restrict__ q_pool,
    const int32_t *__restrict__ p_index, const int32_t *__restrict__ q_index,
    const int32_t *__restrict__ drafts, int gamma, int V, int64_t np, int64_t nq, float cp,
    float cq, const PoolStat *__restrict__ pstat, RowStats *stats, float *alpha_ws,
    float *__restrict__ alpha_out, int64_t i) {
  const int64_t bk = i / gamma, j = i - bk * gamma;
  const int32_t pi = p_index[bk * (gamma + 1) + j];
  const int32_t qi = kGreedy ? 0 : q_index[i];
  const int32_t x = drafts[i];
  float a = __builtin_nanf("");
  RowStats st{kNegInf, __builtin_nanf(""), 0.0f, 1.0f};
  if (pi >= 0 && pi < np && (kGreedy || (qi >= 0 && qi < nq))) {
    const PoolStat ps = pstat[pi];
    const PoolStat qs = kGreedy ? PoolStat{0.0f, 1.0f} : pstat[np + qi];
    st = RowStats{ps.m, ps.s, qs.m, qs.s};
    if (x >= 0 && x < V)
      a = acceptance<kGreedy>(E::at(p_pool + (int64_t)pi * V, x), ps.m, ps.s, cp,
                              kGreedy ? 0.0f : E::at(q_pool + (int64_t)qi * V, x), qs.m, qs.s,
                              cq);
  }
  stats[i] = st;
  alpha_ws[i] = a;
  if (alpha_out) alpha_out[i] = a;
}

template <typename E, bool kGreedy>
__global__ __launch_bounds__(kBlock) void kr_alpha_rows(
    const typename E::elem *__restrict__ p_pool, const typename E::elem *__restrict__ q_pool,
    const int32_t *__restrict__ p_index, const int32_t *__restrict__ q_index,
    const int32_t *__restrict__ drafts, int64_t n, int gamma, int V, int64_t np, int64_t nq,
    float cp, float cq, const PoolStat *__restrict__ pstat, RowStats *__restrict__ stats,
    float *__restrict__ alpha_ws, float *__restrict__ alpha_out) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;  // (b, k, j < gamma)
  if (i >= n) return;
  alpha_row<E, kGreedy>(p_pool, q_pool, p_index, q_index, drafts, gamma, V, np, nq, cp, cq, pstat,
                        stats, alpha_ws, alpha_out, i);
}

}  // namespace svd
