// kr_beam.hpp -- the beam search of the causal-consistency path search.
//
// DiffuSpec section 4.2: a left-to-right beam search over the drafter's
// candidate lattice scores each path by its drafter log-probabilities plus a
// causal-proxy fluency term; section 5.3 settles on beam 3.  The proxy's
// scores come in as a tensor of transition scores between consecutive
// candidates (lambda weighs them).
//
// kr_cps_beam (one 1024-thread workgroup per prefix): expansions (path rank,
//   candidate rank) in fp64, each ranked against all the step's expansions in
//   LDS by a few threads together (the earlier expansion on an exact tie, a NaN
//   score as -inf), the best `beam` kept by rank, backpointers in LDS, paths
//   rebuilt at the end.
#pragma once

#include "kr_cps.hpp"  // kCpsMax, kNegInf

namespace svd {

constexpr int kCpsBeam = 8;      // beam width, at most
constexpr int kCpsMaxG = 1024;   // positions of a beam search, at most
constexpr int kBeamChunk = 16;   // positions of lattice data a beam loads at once
constexpr int kBeamBlock = 1024;  // threads of a beam workgroup (one per prefix)

// n floats from global memory into LDS by the NT threads of the workgroup,
// 16 loads in flight per thread
template <int NT>
__device__ __forceinline__ void copy_to_lds(float *dst, const float *__restrict__ src, int n) {
  const int tid = threadIdx.x;
  for (int t0 = 0; t0 < n; t0 += NT * 16) {
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int t = t0 + k * NT + tid;
      v[k] = t < n ? src[t] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int t = t0 + k * NT + tid;
      if (t < n) dst[t] = v[k];
    }
  }
}

// how many of the n scores es[k0, k0 + n) come before expansion e with score
// v (a larger score, or an equal one at a smaller expansion); n is the same in
// every lane, so the loop unrolls
__device__ __forceinline__ int expansion_rank(const double *es, int k0, int n, double v, int e) {
  int r = 0;
#pragma unroll 4
  for (int m = 0; m < n; ++m) {
    const double x = es[k0 + m];
    r += (x > v) | ((x == v) & (k0 + m < e));
  }
  return r;
}

// One workgroup per prefix.  Expansion (parent rank p, candidate rank i) of a
// step has slot p * kCpsMax + i; slots with i past the position's candidates
// hold NaN, which comes before nothing and is never kept, so slot order is the
// (p, i) order the ranks use.  Every step scores its slots (one thread each),
// then ranks each against all of them with 16 threads per slot (8 past 64
// slots), each counting over its share.
__global__ __launch_bounds__(kBeamBlock) void kr_cps_beam(
    const int32_t *__restrict__ cand, const float *__restrict__ cand_logp,
    const int32_t *__restrict__ n_cand, const int32_t *__restrict__ len,
    const float *__restrict__ fluency, float lambda, int G, int m_max, int beam,
    int32_t *__restrict__ paths, float *__restrict__ path_score, int32_t *__restrict__ path_len) {
  static_assert(kCpsBeam * kCpsMax <= kBeamBlock && kCpsMax == 16, "one thread per slot");
  __shared__ uint8_t bp[kCpsMaxG][kCpsBeam];  // parent rank of rank r at position j
  __shared__ uint8_t ci[kCpsMaxG][kCpsBeam];  // candidate rank of rank r at position j
  __shared__ uint8_t rk[kCpsMaxG][kCpsBeam];  // final path r's candidate rank at position j
  // the beam's path scores and last candidate ranks, by rank: step j reads
  // buffer j % 2 and writes the other
  __shared__ double sc[2][kCpsBeam];
  __shared__ int pc[2][kCpsBeam];
  __shared__ double es[kCpsBeam * kCpsMax];  // the step's expansion scores
  // the lattice of kBeamChunk positions at a time, loaded together
  __shared__ int nc_s[kBeamChunk];
  __shared__ float lp_s[kBeamChunk * kCpsMax];
  __shared__ float fl_s[kBeamChunk * kCpsMax * kCpsMax];
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  int L = len[b];
  // inputs the search cannot use (a length or a candidate count out of range)
  // leave the prefix without paths
  bool ok = L >= 1 && L <= G;
  bool bad = false;
  for (int j = tid; j < (ok ? L : 0); j += kBeamBlock) {
    const int n = n_cand[b * G + j];
    bad |= n < 1 || n > m_max;
  }
  ok = ok && !__syncthreads_or(bad);
  int nb = 1;
  if (tid == 0) {
    sc[0][0] = 0.0;
    pc[0][0] = 0;
  }
  __syncthreads();
  for (int j = 0; ok && j < L; ++j) {
    const int jj = j % kBeamChunk, cur = j & 1;
    if (jj == 0) {  // the next chunk of positions into LDS
      const int n = min(kBeamChunk, L - j);
      const int64_t o0 = b * G + j;
      if (tid < n) nc_s[tid] = n_cand[o0 + tid];
      copy_to_lds<kBeamBlock>(lp_s, cand_logp + o0 * m_max, n * m_max);
      if (fluency) copy_to_lds<kBeamBlock>(fl_s, fluency + o0 * m_max * m_max, n * m_max * m_max);
      __syncthreads();
    }
    const int nc = nc_s[jj];
    const int ns = nb * kCpsMax;  // slots
    // a NaN score of an expansion ranks as -inf, so the ranks of the
    // expansions are a permutation
    if (tid < ns) {
      const int p = tid / kCpsMax, i = tid % kCpsMax;
      double v = __builtin_nan("");
      if (i < nc) {
        const int prev = j == 0 ? 0 : pc[cur][p];
        const double f = fluency ? (double)fl_s[(jj * m_max + prev) * m_max + i] : 0.0;
        v = sc[cur][p] + (double)lp_s[jj * m_max + i] + (double)lambda * f;
        v = v != v ? -INFINITY : v;
      }
      es[tid] = v;
    }
    __syncthreads();
    const int ne = nb * nc, keep = ne < beam ? ne : beam;
    // slot e's T threads are adjacent lanes of one wave
    const int sh = ns <= 64 ? 4 : 3, T = 1 << sh;
    const int e = tid >> sh, part = tid & (T - 1);
    const int per = ns >> sh;  // a multiple of 2
    double v = 0.0;
    int r = 0;
    if (e < ns) {
      v = es[e];
      r = expansion_rank(es, part * per, per, v, e);
    }
    r = group_sum(r, T);
    // an expansion ranked below keep takes that slot of the new beam
    if (part == 0 && e < ns && e % kCpsMax < nc && r < keep) {
      const int p = e / kCpsMax, i = e % kCpsMax;
      sc[cur ^ 1][r] = v;
      pc[cur ^ 1][r] = i;
      bp[j][r] = (uint8_t)p;
      ci[j][r] = (uint8_t)i;
    }
    nb = keep;
    __syncthreads();  // also orders this step's reads of es before the next step's writes
  }
  // rebuild the paths: each live rank follows its backpointers in LDS and
  // records its candidate ranks, then the workgroup gathers the tokens
  const int live_n = ok ? nb : 0;
  if (tid < live_n) {
    int rr = tid;
    for (int j = L - 1; j >= 0; --j) {
      rk[j][tid] = ci[j][rr];
      rr = bp[j][rr];
    }
  }
  __syncthreads();
  for (int t = tid; t < beam * G; t += kBeamBlock) {
    const int r = t / G, j = t - r * G;
    int32_t tok = -1;
    if (r < live_n && j < L) tok = cand[(b * G + j) * m_max + rk[j][r]];
    paths[(b * beam + r) * (int64_t)G + j] = tok;
  }
  if (tid < beam) {
    const bool live = tid < live_n;
    path_score[b * beam + tid] = live ? (float)sc[L & 1][tid] : kNegInf;
    path_len[b * beam + tid] = live ? L : 0;
  }
}

}  // namespace svd
