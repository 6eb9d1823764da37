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
//   (logit descending, index ascending), the order of decreasing probability,
//   compared as one unsigned 64-bit key.  One pass keeps the online
//   (max, sum) and each thread's largest logit; the 16th largest of those
//   maxima bounds the row's 16th largest from below; every token at or above
//   the bound (a few dozen) goes into an LDS list, and each listed token's
//   rank is the count of listed keys above its own.  A bf16 row of at most
//   kLatticeRegVecs vectors per thread is held in registers and read once,
//   its bound taken from the first vectors while the rest arrive; other rows
//   are streamed twice.  If more than kCandCap tokens tie at the bound,
//   per-thread sorted lists over the whole row are merged instead.  The first
//   lanes then turn the 16 best into probabilities and cut at tau.
// kr_lattice_len (one thread per prefix): the lattice length (first position
//   whose best token is EOS, included) and the cleared tail.
// The beam search over the lattice is in kr_beam.hpp.
#pragma once

#include "kr_rowstats.hpp"  // row_ms helpers, kSplitBlock

namespace svd {

constexpr int kCpsMax = 16;      // candidates per position, at most
constexpr int kNoIndex = 0x7fffffff;

// (va, ia) comes before (vb, ib)
__device__ __forceinline__ bool ahead(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// The same order as one unsigned 64-bit key: a larger key is ahead.  The high
// word maps the logit's bits to an order-preserving unsigned value (-0 counts
// as +0, as the float comparison has it), the low word is the inverted index.
// Key 0 stands for "no token": every real key is larger (the high word of -inf
// is 0x007fffff).  NaN is never keyed.
__device__ __forceinline__ uint64_t rank_key(float v, int i) {
  uint32_t b = __float_as_uint(v + 0.0f);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint32_t)~(uint32_t)i;
}
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t b = (uint32_t)(k >> 32);
  return k ? __uint_as_float((b & 0x80000000u) ? (b & 0x7fffffffu) : ~b) : kNegInf;
}
__device__ __forceinline__ int key_index(uint64_t k) {
  return k ? (int)~(uint32_t)k : kNoIndex;
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

// the sum of x over lanes Tq..Tq+T-1 (T = 16, 8 or 4), by quad permutes and,
// past 4, rotations inside the row of 16 lanes (every lane active)
__device__ __forceinline__ int group_sum(int x, int T) {
  x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);  // lane ^ 1
  x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);  // lane ^ 2
  if (T >= 8) {  // row_ror:n hands lane l the value of lane l - n (mod 16)
    const int lo = __builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, false);  // lane - 4
    const int hi = __builtin_amdgcn_update_dpp(0, x, 0x12C, 0xF, 0xF, false);  // lane + 4
    x += (threadIdx.x & 4) ? lo : hi;
  }
  if (T == 16) x += __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);  // lane +- 8
  return x;
}

// row flags written by kr_lattice for kr_lattice_len
enum : uint32_t { kRowInvalid = 1u, kRowEosTop = 2u };

constexpr int kCandCap = 512;  // LDS list of tokens at or above the threshold
// vectors per thread of a row held in registers from which its bound is taken
constexpr int kLatticeBoundVecs = 10;
// keys each wave keeps for the bound of a row held in registers
constexpr int kLatticeWaveKeep = 4;
constexpr int kLatticeMaxSlices = 64;  // slices of one row (one per lane of the merge)

// visit the logits of a row with kRowBlock threads: f(index, value)
// Visit z[0, n) with NT threads: f(index, value); kLatticeUnroll 16-byte
// loads in flight per thread on the vector path.
constexpr int kLatticeUnroll = 4;

template <typename E, bool kVec, int NT, typename F>
__device__ __forceinline__ void visit_row(const typename E::elem *z, int n, F &&f) {
  const int tid = threadIdx.x;
  if constexpr (kVec) {
    constexpr int P = E::kPerVec, U = kLatticeUnroll;
    const vec16 *vz = reinterpret_cast<const vec16 *>(z);
    const int nv = n / P;
    int i = tid;
    for (; i + (U - 1) * NT < nv; i += U * NT) {
      vec16 w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) w[u] = vz[i + u * NT];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x[P];
        E::unpack(w[u], x);
#pragma unroll
        for (int e = 0; e < P; ++e) f((i + u * NT) * P + e, x[e]);
      }
    }
    for (; i < nv; i += NT) {
      float x[P];
      E::unpack(vz[i], x);
#pragma unroll
      for (int e = 0; e < P; ++e) f(i * P + e, x[e]);
    }
  } else {
    for (int i = tid; i < n; i += NT) f(i, E::at(z, i));
  }
}

// LDS of one workgroup finding a row's (or slice's) 16 best tokens.  Each
// wave keeps its KEEP best thread keys (16: the 16th largest of what the waves
// keep is the 16th largest of all threads' keys; fewer: still a lower bound,
// as any subset's 16th largest is); H > 0: the largest logit of each of the
// first H vectors that every thread holds.
template <int NT, int H, int KEEP = kCpsMax>
struct LatticeLds {
  static constexpr int NW = NT / 64;
  static constexpr int NE = NW * KEEP;  // the keys the waves keep
  static constexpr int T = NT / NE;     // threads ranking one of them
  static constexpr int PER = NE / T;    // keys each of those threads compares
  static_assert(NE >= kCpsMax && T * NE == NT && T <= 64, "a bound needs 16 kept keys");
  float ms[2 * NW + 2];                 // block_ms partials, then the (max, sum)
  uint64_t ak[NT];                      // every thread's best key; later the merge's lists
  // wave w's kept keys by rank at entry w * KEEP + rank, each group of PER
  // entries padded by two keys, so that the T readers of one rank step use
  // different LDS banks
  uint64_t wk[NE + 2 * T];
  uint64_t ck[kCandCap];  // the keys of the tokens at or above the bound
  uint64_t sk[kCpsMax];   // the 16 best of those, by rank
  float vmx[H > 0 ? H * NT : 1];
  int n_found;
  float thr;
  __device__ static int slot(int e) { return e + 2 * (e / PER); }
};

// Clears the candidate ranks and count and sets the bound to -inf; a barrier
// before their first use orders this.  (Each wave clears its own rank slots
// in wave_rank16.)
template <class L>
__device__ __forceinline__ void lattice_lds_init(L &sh) {
  const int tid = threadIdx.x;
  if (tid < kCpsMax) sh.sk[tid] = 0;
  if (tid == 0) {
    sh.thr = kNegInf;  // fewer than 16 keyed tokens: all of them
    sh.n_found = 0;
  }
}

// The 16th largest of the threads' keys (key 0: no token) bounds the 16th
// largest logit of the tokens they were taken from, and so of any set holding
// those tokens, from below: 16 distinct tokens reach it.  Each wave ranks its
// 64 keys against each other and keeps its 16 best in rank slots; then four
// threads rank each of those NE against a quarter of them each.  Keys are
// unique (they hold the token index).  Returns the bound's logit in every
// thread (-inf with fewer than 16 keyed tokens).
// The first step, within each wave (no workgroup barrier: a wave reads only
// the keys its own lanes wrote, and its LDS accesses run in program order).
template <class L>
__device__ __forceinline__ void wave_rank16(L &sh, uint64_t key) {
  constexpr int KEEP = L::NE / L::NW;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (lane < KEEP) sh.wk[L::slot(w * KEEP + lane)] = 0;
  sh.ak[tid] = key;
  __builtin_amdgcn_wave_barrier();
  if (key) {
    int r = 0;
#pragma unroll 16
    for (int k = w * 64; k < w * 64 + 64; ++k) r += sh.ak[k] > key;
    if (r < KEEP) sh.wk[L::slot(w * KEEP + r)] = key;
  }
}

// The second step, after a workgroup barrier that follows every wave's first
// step; returns the bound with a barrier after it.
template <class L>
__device__ __forceinline__ float merge_rank16(L &sh) {
  const int tid = threadIdx.x;
  {
    const int e = tid / L::T, part = tid % L::T;  // NE entries, T threads each
    const uint64_t ke = sh.wk[L::slot(e)];
    const uint64_t *qk = sh.wk + L::slot(part * L::PER);
    int r = 0;
#pragma unroll 16
    for (int k = 0; k < L::PER; ++k) r += qk[k] > ke;
#pragma unroll
    for (int off = 1; off < L::T; off <<= 1) r += __shfl_xor(r, off, 64);
    if (part == 0 && ke && r == kCpsMax - 1) sh.thr = key_value(ke);
  }
  __syncthreads();
  return sh.thr;
}

template <class L>
__device__ __forceinline__ float lattice_bound(L &sh, uint64_t key) {
  wave_rank16(sh, key);
  __syncthreads();
  return merge_rank16(sh);
}

// Appends the token (index i, logit x) to the candidate list when it reaches
// the bound (past kCandCap only counted).
template <class L>
__device__ __forceinline__ void lattice_take(L &sh, float thr, int i, float x) {
  if (x >= thr) {
    const int k = atomicAdd(&sh.n_found, 1);
    if (k < kCandCap) sh.ck[k] = rank_key(x, i);
  }
}

// The 16 best of the nf listed candidates, in lanes 0..15 of wave 0 (bv, bi);
// other waves return with undefined values.  When more than kCandCap tokens
// reached the bound (many ties at it), per-thread sorted lists over the
// whole set are merged instead: restream(f) calls f(index, logit) on every
// token of this thread's share.
template <class L, class Restream>
__device__ __forceinline__ void lattice_top16(L &sh, int nf, Restream &&restream, float &bv,
                                              int &bi) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (nf > kCandCap) {
    float tv[kCpsMax];
    int ti[kCpsMax];
#pragma unroll
    for (int k = 0; k < kCpsMax; ++k) {
      tv[k] = kNegInf;
      ti[k] = kNoIndex;
    }
    restream([&](int i, float x) { top_insert(tv, ti, x, i); });
    float v16;
    int i16;
    wave_pop16<kCpsMax>(tv, ti, v16, i16);
    if (lane < kCpsMax) sh.ak[w * kCpsMax + lane] = i16 != kNoIndex ? rank_key(v16, i16) : 0;
  } else {
    // every listed token counts the ones ahead of it, 16 adjacent threads per
    // token over every 16th key, summed by DPP; the 16 best take their rank
    // slots (the trip counts are the same in every lane: the sums need them all)
    constexpr int kPer = L::NW * 4;  // tokens per round
    for (int t0 = 0; t0 < nf; t0 += kPer) {
      const int t = t0 + (tid >> 4), part = tid & 15;
      const uint64_t kt = t < nf ? sh.ck[t] : 0;
      int r = 0;
      for (int k = part; k < nf; k += 16) r += sh.ck[k] > kt;
      r = group_sum(r, 16);
      if (part == 0 && t < nf && r < kCpsMax) sh.sk[r] = kt;
    }
  }
  __syncthreads();
  if (w != 0) return;
  if (nf > kCandCap) {
    constexpr int NL = L::NW * kCpsMax;  // the waves' lists
    constexpr int PER = (NL + 63) / 64;
    float lv[PER];
    int li[PER];
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      const int k = PER * lane + t;
      const uint64_t kk = k < NL ? sh.ak[k] : 0;
      lv[t] = key_value(kk);
      li[t] = key_index(kk);
    }
    wave_pop16<PER>(lv, li, bv, bi);
  } else {
    const uint64_t kk = lane < kCpsMax ? sh.sk[lane] : 0;
    bv = key_value(kk);
    bi = key_index(kk);
  }
}

// The 16 best (logit, index) pairs of z[lo, hi) and the slice's (max, sum),
// by NT threads streaming the slice from memory: one pass for the (max, sum)
// and each thread's largest logit, the bound from those, a second pass that
// lists the tokens at or above it.  Results: (m, s) and, in lanes 0..15 of
// wave 0, the r-th best pair in (bv, bi); other threads return with
// undefined values.
template <typename E, bool kVec, int NT>
__device__ __forceinline__ void lattice_slice(const typename E::elem *row, int lo, int hi, float c,
                                              float &m_out, float &s_out, float &bv, int &bi) {
  using L = LatticeLds<NT, 0>;
  __shared__ L sh;
  const typename E::elem *z = row + lo;  // 16-byte aligned when kVec
  const int n = hi - lo;
  const int tid = threadIdx.x;
  lattice_lds_init(sh);
  float m = kNegInf, s = 0.0f, tmax = kNegInf;
  int tidx = kNoIndex;
  if constexpr (kVec) {  // whole vectors (the slice is one), kLatticeUnroll loads in flight
    constexpr int P = E::kPerVec, U = kLatticeUnroll;
    const vec16 *vz = reinterpret_cast<const vec16 *>(z);
    const int nv = n / P;
    auto fold = [&](const vec16 &wv16, int i) {
      float x[P];
      E::unpack(wv16, x);
      ms_fold<P>(m, s, x, c);
#pragma unroll
      for (int e = 0; e < P; ++e)
        if (ahead(x[e], lo + i * P + e, tmax, tidx)) {
          tmax = x[e];
          tidx = lo + i * P + e;
        }
    };
    int i = tid;
    for (; i + (U - 1) * NT < nv; i += U * NT) {
      vec16 w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) w[u] = vz[i + u * NT];  // kept for the second pass: cached
#pragma unroll
      for (int u = 0; u < U; ++u) fold(w[u], i + u * NT);
    }
    for (; i < nv; i += NT) fold(vz[i], i);
  } else {
    for (int i = tid; i < n; i += NT) {
      float x = E::at(z, i);
      ms_fold<1>(m, s, &x, c);
      if (ahead(x, lo + i, tmax, tidx)) {
        tmax = x;
        tidx = lo + i;
      }
    }
  }
  block_ms<L::NW>(m, s, c, sh.ms);  // valid in thread 0
  if (tid == 0) {
    sh.ms[2 * L::NW] = m;
    sh.ms[2 * L::NW + 1] = s;
  }
  const float thr = lattice_bound(sh, tidx != kNoIndex ? rank_key(tmax, tidx) : 0);
  visit_row<E, kVec, NT>(z, n, [&](int i, float x) { lattice_take(sh, thr, lo + i, x); });
  __syncthreads();
  const int nf = sh.n_found;
  lattice_top16(sh, nf, [&](auto &&f) {
    visit_row<E, kVec, NT>(z, n, [&](int i, float x) { f(lo + i, x); });
  }, bv, bi);
  m_out = sh.ms[2 * L::NW];
  s_out = sh.ms[2 * L::NW + 1];
}

// A whole 16-byte row of at most R vectors per thread, held in registers and
// read from memory once, with nontemporal loads.  Every load is issued at the
// start, a thread past the row's end re-reading its last vector (the folds
// skip it; the row holds at least one vector): loads under a condition would
// make the first fold wait for all of them instead of for each vector as it
// arrives.  Each wave works on until a single workgroup barrier: it folds
// every vector into its (max, sum) as it arrives and keeps each vector's
// largest logit in LDS, ranks the best keys of its threads' first H vectors
// among themselves (a bound from part of the row holds for all of it), and
// leaves its (max, sum).  After the barrier the waves' 16 best give the bound,
// the held vectors whose largest logit reaches it are listed, and wave 0
// merges the waves' (max, sum) in wave order, the order of the streaming
// form's reduction.  Results as lattice_slice's.
template <typename E, int NT, int R>
__device__ __forceinline__ void lattice_row_regs(const typename E::elem *z, int n, float c,
                                                 float &m_out, float &s_out, float &bv, int &bi) {
  constexpr int P = E::kPerVec;
  constexpr int H = kLatticeBoundVecs < R ? kLatticeBoundVecs : R;
  using L = LatticeLds<NT, R, kLatticeWaveKeep>;
  __shared__ L sh;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const vec16 *vz = reinterpret_cast<const vec16 *>(z);
  const int nv = n / P;
  vec16 buf[R];
#pragma unroll
  for (int r = 0; r < R; ++r) buf[r] = __builtin_nontemporal_load(vz + min(tid + r * NT, nv - 1));
  lattice_lds_init(sh);

  // every vector as it arrives: (max, sum) and its largest logit; over the
  // first H, the thread's best, tracked per vector (its first vector holding
  // the largest logit; NaN never wins) and located inside it afterwards, which
  // keeps the (logit descending, index ascending) order
  float m = kNegInf, s = 0.0f, tmax = kNegInf;
  int tvec = -1;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (tid + r * NT < nv) {
      float x[P];
      E::unpack(buf[r], x);
      ms_fold<P>(m, s, x, c);
      float vm = x[0];
#pragma unroll
      for (int e = 1; e < P; ++e) vm = fmaxf(vm, x[e]);
      sh.vmx[r * NT + tid] = vm;  // NaN only for a vector of NaN
      if (r < H && vm == vm && (tvec < 0 || vm > tmax)) {
        tmax = vm;
        tvec = r;
      }
    }
    if (r == H - 1) {  // the thread's best of the first H vectors, ranked in the wave
      int tidx = kNoIndex;
#pragma unroll
      for (int q = 0; q < H; ++q) {
        if (q == tvec) {
          float y[P];
          E::unpack(buf[q], y);
          int e0 = P - 1;
#pragma unroll
          for (int e = P - 1; e >= 0; --e)
            if (y[e] == tmax) e0 = e;
          tidx = (tid + q * NT) * P + e0;
        }
      }
      wave_rank16(sh, tidx != kNoIndex ? rank_key(tmax, tidx) : 0);
    }
  }
  // this wave's (max, sum), by the butterfly of block_ms
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float mo = __shfl_xor(m, off, 64);
    const float so = __shfl_xor(s, off, 64);
    ms_merge(m, s, mo, so, c);
  }
  if (lane == 0) {
    sh.ms[2 * w] = m;
    sh.ms[2 * w + 1] = s;
  }
  __syncthreads();
  const float thr = merge_rank16(sh);

  // the held vectors whose largest logit reaches the bound
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = tid + r * NT;
    if (i < nv && sh.vmx[r * NT + tid] >= thr) {
      float x[P];
      E::unpack(buf[r], x);
#pragma unroll
      for (int e = 0; e < P; ++e) lattice_take(sh, thr, i * P + e, x[e]);
    }
  }
  __syncthreads();
  const int nf = sh.n_found;
  // (the rare many-ties merge streams the row again, which keeps every
  // register access in a fully unrolled loop)
  lattice_top16(sh, nf, [&](auto &&f) { visit_row<E, true, NT>(z, n, f); }, bv, bi);
  if (w != 0) return;
  float v[2 * L::NW];  // (all read at once; the merge keeps the wave order)
#pragma unroll
  for (int k = 0; k < 2 * L::NW; ++k) v[k] = sh.ms[k];
  m = v[0];
  s = v[1];
#pragma unroll
  for (int k = 1; k < L::NW; ++k) ms_merge(m, s, v[2 * k], v[2 * k + 1], c);
  m_out = m;
  s_out = s;
}

// Wave 0 with the row's 16 best pairs (lane r holds the r-th in bv, bi) and its
// (max, sum): probabilities, their running sum in rank order, the cut at tau,
// the outputs of the row.
__device__ __forceinline__ void lattice_finish(int64_t row, float rm, float rs, float bv, int bi,
                                               float c, float tau, int m_max, int eos,
                                               int32_t *__restrict__ cand,
                                               float *__restrict__ cand_logp,
                                               int32_t *__restrict__ n_cand,
                                               uint32_t *__restrict__ flags) {
  const int lane = threadIdx.x & 63;
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
  const int n = hit ? __ffsll((unsigned long long)hit) : __popcll(avail);  // first rank reaching tau, + 1
  if (lane < m_max) {
    const int64_t o = row * m_max + lane;
    cand[o] = lane < n ? bi : -1;
    cand_logp[o] = lane < n ? lg2 * 0.6931471805599453f : kNegInf;
  }
  const int b0 = __shfl(bi, 0, 64);
  if (lane == 0) {
    n_cand[row] = n;
    uint32_t f = 0u;
    if (rs != rs || rm == kNegInf) f |= kRowInvalid;
    if (eos >= 0 && b0 == eos) f |= kRowEosTop;
    flags[row] = f;
  }
}

// Vectors per thread a whole-row workgroup holds in registers: a bf16 row of
// up to 19 * 1024 * 8 = 155648 tokens (a Qwen2.5-size vocabulary) is read
// once; longer rows and fp32 rows stream twice.
constexpr int kLatticeRegVecs = 19;

template <typename E, bool kVec>
constexpr int lattice_regs() {
  return kVec && sizeof(typename E::elem) == 2 ? kLatticeRegVecs : 0;
}

// one workgroup per drafter row; R > 0: the row is held in registers (the
// host launches this form only when it has at most R vectors per thread)
template <typename E, bool kVec, int R>
__global__ __launch_bounds__(kRowBlock) void kr_lattice(
    const typename E::elem *__restrict__ q, int V, float c, float tau, int m_max, int eos,
    int32_t *__restrict__ cand, float *__restrict__ cand_logp, int32_t *__restrict__ n_cand,
    uint32_t *__restrict__ flags) {
  const int64_t row = blockIdx.x;  // b * G + j
  float m, s, bv;
  int bi;
  if constexpr (R > 0)
    lattice_row_regs<E, kRowBlock, R>(q + row * (int64_t)V, V, c, m, s, bv, bi);
  else
    lattice_slice<E, kVec, kRowBlock>(q + row * (int64_t)V, 0, V, c, m, s, bv, bi);
  if (threadIdx.x >= 64) return;
  lattice_finish(row, m, s, bv, bi, c, tau, m_max, eos, cand, cand_logp, n_cand, flags);
}

// Split rows, as for the row statistics: slice sl of row r in workgroup
// r * S + sl, a record of the slice's (max, sum) and 16 best pairs, then one
// wave per row merges the S records.
struct LatticePart {
  float m, s;
  float v[kCpsMax];
  int i[kCpsMax];
};

template <typename E, bool kVec>
__global__ __launch_bounds__(kSplitBlock) void kr_lattice_split(
    const typename E::elem *__restrict__ q, int V, float c, int S, int slice,
    LatticePart *__restrict__ part) {
  const int64_t r = blockIdx.x / S;
  const int sl = (int)(blockIdx.x - r * S);
  const int lo = sl * slice, hi = min(V, lo + slice);  // slice: whole vectors
  float m, s, bv;
  int bi;
  lattice_slice<E, kVec, kSplitBlock>(q + r * (int64_t)V, lo, hi, c, m, s, bv, bi);
  if (threadIdx.x >= kCpsMax) return;
  LatticePart *o = part + blockIdx.x;
  if (threadIdx.x == 0) {
    o->m = m;
    o->s = s;
  }
  o->v[threadIdx.x] = bv;
  o->i[threadIdx.x] = bi;
}

__global__ __launch_bounds__(kBlock) void kr_lattice_combine(
    int64_t rows, float c, float tau, int m_max, int eos, int S,
    const LatticePart *__restrict__ part, int32_t *__restrict__ cand,
    float *__restrict__ cand_logp, int32_t *__restrict__ n_cand, uint32_t *__restrict__ flags) {
  const int64_t row = ((int64_t)blockIdx.x * kBlock + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;  // whole waves
  // lane sl holds slice sl's sorted list (S <= 64)
  float lv[kCpsMax];
  int li[kCpsMax];
  float m = kNegInf, s = 0.0f;
  if (lane < S) {
    const LatticePart *pp = part + row * S + lane;
    m = pp->m;
    s = pp->s;
#pragma unroll
    for (int k = 0; k < kCpsMax; ++k) {
      lv[k] = pp->v[k];
      li[k] = pp->i[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < kCpsMax; ++k) {
      lv[k] = kNegInf;
      li[k] = kNoIndex;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
    ms_merge(m, s, __shfl_xor(m, off, 64), __shfl_xor(s, off, 64), c);
  float bv;
  int bi;
  wave_pop16<kCpsMax>(lv, li, bv, bi);
  lattice_finish(row, m, s, bv, bi, c, tau, m_max, eos, cand, cand_logp, n_cand, flags);
}

// One wave per prefix: the first row flagged invalid or with EOS on top.
__global__ __launch_bounds__(kBlock) void kr_lattice_len(const uint32_t *__restrict__ flags,
                                                         int64_t B, int G, int m_max,
                                                         int32_t *__restrict__ cand,
                                                         float *__restrict__ cand_logp,
                                                         int32_t *__restrict__ n_cand,
                                                         int32_t *__restrict__ len) {
  const int64_t b = ((int64_t)blockIdx.x * kBlock + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (b >= B) return;  // whole waves
  int first = G;  // first flagged row
  uint32_t ff = 0u;
  for (int j0 = 0; j0 < G && first == G; j0 += 64) {
    const int j = j0 + lane;
    const uint32_t f = j < G ? flags[b * G + j] : 0u;
    const uint64_t hit = __ballot(f != 0u);
    if (hit) {
      const int k = __ffsll((unsigned long long)hit) - 1;
      first = j0 + k;
      ff = __shfl(f, k, 64);
    }
  }
  const int L = first == G ? G : ((ff & kRowInvalid) ? -1 : first + 1);
  const bool eos_end = first < G && !(ff & kRowInvalid);
  if (lane == 0) len[b] = L;
  for (int j = lane; j < G; j += 64) {
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

}  // namespace svd
