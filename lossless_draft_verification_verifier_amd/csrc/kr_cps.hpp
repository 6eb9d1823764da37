// kr_cps.hpp -- causal-consistency path search over the drafter's lattice.
//
// DiffuSpec section 4.2: the diffusion drafter's per-position candidates form
// a lattice; each position keeps its most probable tokens until their
// cumulative mass reaches tau (at most m_max), the lattice stops at the first
// EOS, and a left-to-right beam search scores paths by drafter confidence plus
// a causal-proxy fluency (section 5.3 settles on beam 3, M_max 15, tau 0.8).
// The proxy's scores need a model, so they come in as a tensor of transition
// scores between consecutive candidates.
//
// kr_lattice (one workgroup per drafter row): candidates are ordered by
//   (logit descending, index ascending), the order of decreasing probability.
//   One streaming pass keeps the online (max, sum) and each thread's largest
//   logit; the 16th largest of those maxima bounds the row's 16th largest from
//   below; a second pass puts every token at or above the bound (a few dozen)
//   into an LDS list, which wave 0 sorts and pops.  If more than kCandCap
//   tokens tie at the bound, per-thread sorted lists over the whole row are
//   merged instead.  The first lanes then turn the 16 best into probabilities
//   and cut at tau.
// kr_lattice_len (one thread per prefix): the lattice length (first position
//   whose best token is EOS, included) and the cleared tail.
// kr_cps_beam (one wave per prefix): expansions (path rank, candidate rank) in
//   fp64, the best `beam` popped one at a time (the earlier expansion on an
//   exact tie), backpointers in LDS, paths rebuilt at the end.
#pragma once

#include "kr_rowstats.hpp"

namespace svd {

constexpr int kCpsMax = 16;      // candidates per position, at most
constexpr int kCpsBeam = 8;      // beam width, at most
constexpr int kCpsMaxG = 1024;   // positions of a beam search, at most
constexpr int kNoIndex = 0x7fffffff;

// (va, ia) comes before (vb, ib)
__device__ __forceinline__ bool ahead(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// insert into a sorted list of kCpsMax entries (the last one drops out)
__device__ __forceinline__ void top_insert(float (&tv)[kCpsMax], int (&ti)[kCpsMax], float v,
                                           int i) {
  if (!ahead(v, i, tv[kCpsMax - 1], ti[kCpsMax - 1])) return;
  tv[kCpsMax - 1] = v;
  ti[kCpsMax - 1] = i;
#pragma unroll
  for (int k = kCpsMax - 1; k > 0; --k) {
    const bool sw = ahead(tv[k], ti[k], tv[k - 1], ti[k - 1]);
    const float a = tv[k], c = tv[k - 1];
    const int ia = ti[k], ic = ti[k - 1];
    tv[k] = sw ? c : a;
    tv[k - 1] = sw ? a : c;
    ti[k] = sw ? ic : ia;
    ti[k - 1] = sw ? ia : ic;
  }
}

// the wave's best entry among the lanes' heads (v, i); every lane gets it
__device__ __forceinline__ void wave_best(float &v, int &i) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(v, off, 64);
    const int oi = __shfl_xor(i, off, 64);
    if (ahead(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

// pop the wave's 16 best entries out of per-lane sorted lists of N entries;
// lane r < 16 receives the r-th best
template <int N>
__device__ __forceinline__ void wave_pop16(float (&lv)[N], int (&li)[N], float &out_v,
                                           int &out_i) {
  const int lane = threadIdx.x & 63;
  out_v = kNegInf;
  out_i = kNoIndex;
#pragma unroll 1
  for (int r = 0; r < kCpsMax; ++r) {
    float v = lv[0];
    int i = li[0];
    wave_best(v, i);
    if (lane == r) {
      out_v = v;
      out_i = i;
    }
    if (li[0] == i && lv[0] == v && i != kNoIndex) {  // this lane held it: shift its list
#pragma unroll
      for (int k = 0; k < N - 1; ++k) {
        lv[k] = lv[k + 1];
        li[k] = li[k + 1];
      }
      lv[N - 1] = kNegInf;
      li[N - 1] = kNoIndex;
    }
  }
}

// row flags written by kr_lattice for kr_lattice_len
enum : uint32_t { kRowInvalid = 1u, kRowEosTop = 2u };

constexpr int kCandCap = 512;  // LDS list of tokens at or above the threshold

// visit the logits of a row with kRowBlock threads: f(index, value)
template <typename E, bool kVec, typename F>
__device__ __forceinline__ void visit_row(const typename E::elem *z, int V, F &&f) {
  const int tid = threadIdx.x;
  if constexpr (kVec) {
    constexpr int P = E::kPerVec;
    const vec16 *vz = reinterpret_cast<const vec16 *>(z);
    for (int i = tid; i < V / P; i += kRowBlock) {
      float x[P];
      E::unpack(vz[i], x);
#pragma unroll
      for (int e = 0; e < P; ++e) f(i * P + e, x[e]);
    }
  } else {
    for (int i = tid; i < V; i += kRowBlock) f(i, E::at(z, i));
  }
}

template <typename E, bool kVec>
__global__ __launch_bounds__(kRowBlock) void kr_lattice(
    const typename E::elem *__restrict__ q, int V, float c, float tau, int m_max, int eos,
    int32_t *__restrict__ cand, float *__restrict__ cand_logp, int32_t *__restrict__ n_cand,
    uint32_t *__restrict__ flags) {
  constexpr int NW = kRowBlock / 64;
  __shared__ float lds[2 * NW];
  __shared__ float wv[NW * kCpsMax];
  __shared__ int wi[NW * kCpsMax];
  __shared__ float cv[kCandCap];
  __shared__ int cix[kCandCap];
  __shared__ int n_found;
  __shared__ float thr_s;
  const int64_t row = blockIdx.x;  // b * G + j
  const typename E::elem *z = q + row * (int64_t)V;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // 1. one streaming pass: (max, sum) of the row and this thread's largest logit
  float m = kNegInf, s = 0.0f, tmax = kNegInf;
  int tidx = kNoIndex;
  if constexpr (kVec) {
    constexpr int P = E::kPerVec;
    const vec16 *vz = reinterpret_cast<const vec16 *>(z);
    for (int i = tid; i < V / P; i += kRowBlock) {
      float x[P];
      E::unpack(stream_load(vz + i), x);
      ms_fold<P>(m, s, x, c);
#pragma unroll
      for (int e = 0; e < P; ++e)
        if (ahead(x[e], i * P + e, tmax, tidx)) {
          tmax = x[e];
          tidx = i * P + e;
        }
    }
  } else {
    for (int i = tid; i < V; i += kRowBlock) {
      float x = E::at(z, i);
      ms_fold<1>(m, s, &x, c);
      if (ahead(x, i, tmax, tidx)) {
        tmax = x;
        tidx = i;
      }
    }
  }
  block_ms<NW>(m, s, c, lds);  // valid in thread 0
  if (tid == 0) {
    lds[0] = m;
    lds[1] = s;
    n_found = 0;
  }
  // 2. the 16th largest of the threads' maxima bounds the row's 16th largest
  //    logit from below: every one of the row's 16 best is at least that
  {
    float lv[1] = {tmax};
    int li[1] = {tidx};
    float v16;
    int i16;
    wave_pop16<1>(lv, li, v16, i16);
    if (lane < kCpsMax) {
      wv[w * kCpsMax + lane] = v16;
      wi[w * kCpsMax + lane] = i16;
    }
  }
  __syncthreads();
  if (w == 0) {
    float lv[4];
    int li[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      lv[t] = wv[4 * lane + t];
      li[t] = wi[4 * lane + t];
    }
    float v16;
    int i16;
    wave_pop16<4>(lv, li, v16, i16);
    const float t16 = __shfl(v16, kCpsMax - 1, 64);
    const int n16 = __shfl(i16, kCpsMax - 1, 64);
    if (lane == 0) thr_s = n16 == kNoIndex ? kNegInf : t16;  // fewer than 16 tokens: all
  }
  __syncthreads();
  // 3. second pass: every token at or above the bound into an LDS list
  const float thr = thr_s;
  visit_row<E, kVec>(z, V, [&](int i, float x) {
    if (x >= thr) {
      const int k = atomicAdd(&n_found, 1);
      if (k < kCandCap) {
        cv[k] = x;
        cix[k] = i;
      }
    }
  });
  __syncthreads();
  const int nf = n_found;
  if (nf > kCandCap) {
    // many tokens tie at the bound: sorted per-thread lists over the whole row
    float tv[kCpsMax];
    int ti[kCpsMax];
#pragma unroll
    for (int k = 0; k < kCpsMax; ++k) {
      tv[k] = kNegInf;
      ti[k] = kNoIndex;
    }
    visit_row<E, kVec>(z, V, [&](int i, float x) { top_insert(tv, ti, x, i); });
    float v16;
    int i16;
    wave_pop16<kCpsMax>(tv, ti, v16, i16);
    if (lane < kCpsMax) {
      wv[w * kCpsMax + lane] = v16;
      wi[w * kCpsMax + lane] = i16;
    }
    __syncthreads();
  }
  if (w != 0) return;
  const float rm = lds[0], rs = lds[1];
  float bv;
  int bi;
  if (nf > kCandCap) {
    float lv[4];
    int li[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      lv[t] = wv[4 * lane + t];
      li[t] = wi[4 * lane + t];
    }
    wave_pop16<4>(lv, li, bv, bi);
  } else {
    // lane l sorts the list entries l, l + 64, ... (at most 8), then the wave pops
    float lv[kCandCap / 64];
    int li[kCandCap / 64];
#pragma unroll
    for (int t = 0; t < kCandCap / 64; ++t) {
      lv[t] = kNegInf;
      li[t] = kNoIndex;
    }
#pragma unroll
    for (int t = 0; t < kCandCap / 64; ++t) {
      const int k = lane + 64 * t;
      if (k < nf) {
        float v = cv[k];
        int i = cix[k];
#pragma unroll
        for (int u = 0; u < kCandCap / 64; ++u) {  // insertion into the sorted list
          if (ahead(v, i, lv[u], li[u])) {
            const float tvv = lv[u];
            const int tii = li[u];
            lv[u] = v;
            li[u] = i;
            v = tvv;
            i = tii;
          }
        }
      }
    }
    wave_pop16<kCandCap / 64>(lv, li, bv, bi);
  }
  // probabilities of the 16 best, their running sum in rank order, the cut at tau
  const bool real = lane < kCpsMax && bi != kNoIndex;
  const float lg2 = (bv - rm) * c - log2f(rs);  // log2 p
  float p = real ? exp2f(lg2) : 0.0f;
  float cum = p;
#pragma unroll
  for (int off = 1; off < kCpsMax; off <<= 1) {  // inclusive scan over lanes 0..15
    const float y = __shfl_up(cum, off, 64);
    if (lane >= off) cum += y;
  }
  const bool reached = real && lane < m_max && cum >= tau;
  const uint64_t hit = __ballot(reached);
  const uint64_t avail = __ballot(real && lane < m_max);
  const int n = hit ? __ffsll((unsigned long long)hit) : __popcll(avail);
  if (lane < m_max) {
    const int64_t o = row * m_max + lane;
    cand[o] = lane < n ? bi : -1;
    cand_logp[o] = lane < n ? lg2 * 0.6931471805599453f : kNegInf;
  }
  if (lane == 0) {
    n_cand[row] = n;
    uint32_t f = 0u;
    if (rs != rs || rm == kNegInf) f |= kRowInvalid;
    if (eos >= 0 && bi == eos) f |= kRowEosTop;
    flags[row] = f;
  }
}

__global__ __launch_bounds__(kBlock) void kr_lattice_len(const uint32_t *__restrict__ flags,
                                                         int64_t B, int G, int m_max,
                                                         int32_t *__restrict__ cand,
                                                         float *__restrict__ cand_logp,
                                                         int32_t *__restrict__ n_cand,
                                                         int32_t *__restrict__ len) {
  const int64_t b = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (b >= B) return;
  int L = G;
  bool eos_end = false;
  for (int j = 0; j < G; ++j) {
    const uint32_t f = flags[b * G + j];
    if (f & kRowInvalid) {
      L = -1;
      break;
    }
    if (f & kRowEosTop) {
      L = j + 1;
      eos_end = true;
      break;
    }
  }
  len[b] = L;
  for (int j = 0; j < G; ++j) {
    const int64_t o = b * G + j;
    int keep = n_cand[o];
    if (L < 0 || j >= L) keep = 0;
    else if (eos_end && j == L - 1) keep = 1;
    if (keep == n_cand[o]) continue;
    n_cand[o] = keep;
    for (int i = keep; i < m_max; ++i) {
      cand[o * m_max + i] = -1;
      cand_logp[o * m_max + i] = kNegInf;
    }
  }
}

// best (score, expansion) over the wave: larger score, then the smaller expansion
__device__ __forceinline__ void wave_best_d(double &s, int &e) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const double os = __shfl_xor(s, off, 64);
    const int oe = __shfl_xor(e, off, 64);
    if (os > s || (os == s && oe < e)) {
      s = os;
      e = oe;
    }
  }
}

__global__ __launch_bounds__(64) void kr_cps_beam(
    const int32_t *__restrict__ cand, const float *__restrict__ cand_logp,
    const int32_t *__restrict__ n_cand, const int32_t *__restrict__ len,
    const float *__restrict__ fluency, float lambda, int G, int m_max, int beam,
    int32_t *__restrict__ paths, float *__restrict__ path_score, int32_t *__restrict__ path_len) {
  __shared__ uint8_t bp[kCpsMaxG][kCpsBeam];  // parent rank of rank r at position j
  __shared__ uint8_t ci[kCpsMaxG][kCpsBeam];  // candidate rank of rank r at position j
  __shared__ double sc[kCpsBeam], nsc[kCpsBeam];
  __shared__ int pc[kCpsBeam], npc[kCpsBeam];
  const int64_t b = blockIdx.x;
  const int lane = threadIdx.x;
  int L = len[b];
  // inputs the search cannot use (a length or a candidate count out of range)
  // leave the prefix without paths
  bool ok = L >= 1 && L <= G;
  bool bad = false;
  for (int j = lane; j < (L >= 1 && L <= G ? L : 0); j += 64) {
    const int n = n_cand[b * G + j];
    bad |= n < 1 || n > m_max;
  }
  ok = ok && !__any(bad);
  int nb = 1;
  if (lane == 0) {
    sc[0] = 0.0;
    pc[0] = 0;
  }
  __syncthreads();
  for (int j = 0; ok && j < L; ++j) {
    const int64_t o = b * G + j;
    const int nc = n_cand[o];
    const int ne = nb * nc;
    double s0 = -INFINITY, s1 = -INFINITY;
    auto score = [&](int e) -> double {
      const int p = e / nc, i = e - p * nc;
      const int prev = j == 0 ? 0 : pc[p];
      const double f = fluency ? (double)fluency[(o * m_max + prev) * m_max + i] : 0.0;
      return sc[p] + (double)cand_logp[o * m_max + i] + (double)lambda * f;
    };
    const int e0 = lane, e1 = lane + 64;
    if (e0 < ne) s0 = score(e0);
    if (e1 < ne) s1 = score(e1);
    bool u0 = e0 >= ne, u1 = e1 >= ne;  // used (or absent)
    const int keep = ne < beam ? ne : beam;
    for (int r = 0; r < keep; ++r) {
      // this lane's best unused expansion, then the wave's
      double s = -INFINITY;
      int e = kNoIndex;
      if (!u0) {
        s = s0;
        e = e0;
      }
      if (!u1 && (e == kNoIndex || s1 > s)) {
        s = s1;
        e = e1;
      }
      wave_best_d(s, e);
      if (e == e0) u0 = true;
      if (e == e1) u1 = true;
      if (lane == 0) {
        const int p = e / nc, i = e - p * nc;
        nsc[r] = s;
        npc[r] = i;
        bp[j][r] = (uint8_t)p;
        ci[j][r] = (uint8_t)i;
      }
    }
    __syncthreads();
    if (lane < keep) {
      sc[lane] = nsc[lane];
      pc[lane] = npc[lane];
    }
    nb = keep;
    __syncthreads();
  }
  // rebuild the paths from the backpointers
  if (lane < beam) {
    int32_t *out = paths + (b * beam + lane) * (int64_t)G;
    const bool live = ok && lane < nb;
    int rr = lane;
    for (int j = G - 1; j >= 0; --j) {
      int32_t tok = -1;
      if (live && j < L) {
        const int i = ci[j][rr];
        tok = cand[(b * G + j) * m_max + i];
        rr = bp[j][rr];
      }
      out[j] = tok;
    }
    path_score[b * beam + lane] = live ? (float)sc[lane] : kNegInf;
    path_len[b * beam + lane] = live ? L : 0;
  }
}

}  // namespace svd
