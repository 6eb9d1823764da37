// svd_device.hpp -- device-side helpers shared by the verification kernels:
// logit loads, the counter-hash uniforms and workgroup reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svd {

constexpr int kBlock = 256;         // threads per workgroup (4 waves of 64)
constexpr int kWaves = kBlock / 64;
constexpr int kDrawSeg = 8192;      // vocabulary segment of the fp64 draw
constexpr int kDrawSegSmall = 1024; // the same for batches too small to fill the GPU
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLowest = -3.40282347e38f;

// 16 bytes of logits as a native vector, so that one buffer load moves it
typedef uint32_t vec16 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Logit element types.  bf16 is carried as its 16-bit pattern; widening to
// fp32 puts it in the upper half of the fp32 word, which is exact.

struct BF16 {
  using elem = uint16_t;
  static constexpr int kPerVec = 8;   // elements per 16-byte load
  __device__ static inline float at(const elem *row, int64_t i) {
    return __uint_as_float((uint32_t)row[i] << 16);
  }
  // unpack one 16-byte vector into 8 floats
  __device__ static inline void unpack(const vec16 &w, float *x) {
    x[0] = __uint_as_float(w.x << 16); x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16); x[3] = __uint_as_float(w.y & 0xffff0000u);
    x[4] = __uint_as_float(w.z << 16); x[5] = __uint_as_float(w.z & 0xffff0000u);
    x[6] = __uint_as_float(w.w << 16); x[7] = __uint_as_float(w.w & 0xffff0000u);
  }
};

struct F32 {
  using elem = float;
  static constexpr int kPerVec = 4;
  __device__ static inline float at(const elem *row, int64_t i) { return row[i]; }
  __device__ static inline void unpack(const vec16 &w, float *x) {
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
  }
};

// ---------------------------------------------------------------------------
// Counter-hash uniforms from the published SplitMix64 output function
// (Steele, Lea and Flood, OOPSLA 2014): one uniform per (seed, prefix row,
// position, purpose), U = (KEY >> 11) * 2^-53.

enum : uint32_t { kAccept = 1, kResidual = 2, kBonus = 3 };

__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ double counter_uniform(uint64_t seed, uint64_t row, uint64_t pos,
                                         uint64_t purpose) {
  uint64_t h = splitmix64(splitmix64(splitmix64(splitmix64(seed) ^ row) ^ pos) ^ purpose);
  return (double)(h >> 11) * 0x1.0p-53;
}

// ---------------------------------------------------------------------------
// exp2 on the transcendental unit.  Terms below 2^-126 of the row maximum
// are irrelevant to every sum here, so the raw instruction is enough.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge two (max, sum) states of an online softmax whose terms are
// exp2((z - max) * c).  Commutative, so butterfly reductions leave the same
// bits in every lane.
__device__ __forceinline__ void ms_merge(float &m, float &s, float mo, float so, float c) {
  float mn = fmaxf(m, mo);
  float a = (m == mn) ? s : s * fast_exp2((m - mn) * c);
  float b = (mo == mn) ? so : so * fast_exp2((mo - mn) * c);
  m = mn;
  s = a + b;
}

// Workgroup-wide reductions over NW waves of 64 lanes: a butterfly inside each
// wave, then the wave results in wave order.  Every one has a fixed order.

// merge of (max, sum); the result is valid in thread 0
template <int NW>
__device__ __forceinline__ void block_ms(float &m, float &s, float c, float *lds /* 2*NW */) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    float mo = __shfl_xor(m, off, 64);
    float so = __shfl_xor(s, off, 64);
    ms_merge(m, s, mo, so, c);
  }
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    lds[2 * w] = m;
    lds[2 * w + 1] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    m = lds[0];
    s = lds[1];
#pragma unroll 1
    for (int i = 1; i < NW; ++i) ms_merge(m, s, lds[2 * i], lds[2 * i + 1], c);
  }
  __syncthreads();
}

template <int NW>
__device__ __forceinline__ float block_max(float v, float *lds /* NW + 1 */) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = lds[0];
#pragma unroll 1
    for (int i = 1; i < NW; ++i) r = fmaxf(r, lds[i]);
    lds[NW] = r;
  }
  __syncthreads();
  const float r = lds[NW];
  __syncthreads();
  return r;  // valid in every thread
}

template <int NW>
__device__ __forceinline__ float block_sum_f(float v, float *lds /* NW + 1 */) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = v + __shfl_xor(v, off, 64);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = lds[0];
#pragma unroll 1
    for (int i = 1; i < NW; ++i) r = r + lds[i];
    lds[NW] = r;
  }
  __syncthreads();
  const float r = lds[NW];
  __syncthreads();
  return r;  // valid in every thread
}

template <int NW>
__device__ __forceinline__ double block_sum_d(double v, double *lds /* NW + 1 */) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = v + __shfl_xor(v, off, 64);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    double r = lds[0];
#pragma unroll 1
    for (int i = 1; i < NW; ++i) r = r + lds[i];
    lds[NW] = r;
  }
  __syncthreads();
  const double r = lds[NW];
  __syncthreads();
  return r;  // valid in every thread
}

template <int NW>
__device__ __forceinline__ int block_max_i(int v, int *lds /* NW + 1 */) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int r = lds[0];
#pragma unroll 1
    for (int i = 1; i < NW; ++i) r = max(r, lds[i]);
    lds[NW] = r;
  }
  __syncthreads();
  const int r = lds[NW];
  __syncthreads();
  return r;  // valid in every thread
}

template <int NW>
__device__ __forceinline__ int block_min_i(int v, int *lds /* NW + 1 */) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off, 64));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int r = lds[0];
#pragma unroll 1
    for (int i = 1; i < NW; ++i) r = min(r, lds[i]);
    lds[NW] = r;
  }
  __syncthreads();
  const int r = lds[NW];
  __syncthreads();
  return r;  // valid in every thread
}

// ---------------------------------------------------------------------------
// Workspace records.

struct RowStats {      // one scored row pair
  float mp, sp;        // raw max logit of the p row, sum of exp2((z - mp) * cp)
  float mq, sq;        // the same for the q row
};

}  // namespace svd
