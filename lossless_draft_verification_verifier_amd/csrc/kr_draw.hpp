// kr_draw.hpp -- the replacement / bonus draw in fp64.
//
// After the first rejection at position L the replacement token comes from the
// normalised residual max(0, p - q) of row pair (k*, L) (SpecDiff-2 section 2;
// DiffuSpec section 3, "Acceptance and rejection"); when every drafted token
// is accepted the bonus token comes from p of row gamma.  A residual without
// mass (p equal to q in double) falls back to p.  The token is the first one
// whose cumulative weight exceeds t = u * Z, so tokens of zero weight are
// never drawn; if rounding leaves no such token, the last token with weight.
//
// The selection has already settled the drawn rows and their statistics
// (DrawDesc).  The rows are recomputed from the logits in fp64, in two
// launches:
//
// kr_draw_pass (prefix, vocabulary segment of SEG tokens), one fp64 pass:
//   residual draw: with the exact row maxima m_p, m_q from the row-statistics
//     kernel, w_p = exp((z_p - m_p)/T_p) and w_q likewise; the segment sums of w_p and
//     w_q give the exact normalisers S_p, S_q.  Whether p_v > q_v, i.e.
//     w_p > (S_p/S_q) w_q, is decided against the fp32 ratio from the
//     row-statistics kernel with a relative margin kClassMargin far above its
//     error, without branches: sure-positive tokens add w_p and w_q to two
//     more segment sums, so sum_v max(0, p_v - q_v) over them is
//     (sum w_p)/S_p - (sum w_q)/S_q.  The rare tokens inside the margin are
//     settled once S_p and S_q are known.  At equal temperatures the ratio
//     p_v / q_v of a token depends only on the logit difference
//     d = z_p - z_q (it is exp((d - m_p + m_q)/T) S_q / S_p up to rounding), and
//     bf16 logits put hundreds of tokens on each difference, so a margin
//     token's difference is its class: tokens with d = 0 go to two more sums,
//     the others are collected in LDS and, when more than kUncCap, merged
//     class by class; a class has one sign, and a token whose own sign could
//     differ from it is within 1e-12 of p_v = q_v, where its weight is below
//     rounding.  At most kUncCap entries (single tokens or classes) are kept
//     per segment.
//   p-row draw (bonus, or greedy rejection): the sums of exp((z - m)/T) with
//     and without the excluded token, m the row max when the row was scored
//     (greedy rejection), else the segment max from a first sweep (bonus row).
// kr_draw_pick (prefix, kPickBlock threads): exact normalisers and segment
//   masses (a segment whose uncertain list overflowed is recomputed here, all
//   threads on one segment), the segment that holds t (a scan over lanes that
//   hold one segment each, or a run of consecutive segments each when there
//   are more than 64), then each thread takes kRun consecutive tokens of that
//   segment into registers and a workgroup prefix sum over the threads' totals
//   locates the token.  The rare fallback (t at or past the total) scans
//   segments from the end for the last token with weight.
// SEG is kDrawSeg, or kDrawSegSmall when the batch has too few prefixes to
// fill the GPU with segments of kDrawSeg tokens.
// Every reduction has a fixed order and the uncertain tokens are summed in
// token order, so the result is deterministic.
#pragma once

#include <type_traits>

#include "kr_select.hpp"

namespace svd {

constexpr int kUncCap = 32;            // uncertain tokens kept per segment
constexpr int kPickBlock = 512;        // threads of a pick workgroup
constexpr int kUncList = 256;          // margin tokens a pass workgroup collects
constexpr int kPickSegs = 256;         // segment records the pick stages in LDS
constexpr int kPickUncSegs = 32;       // segments whose uncertain lists the pick stages
constexpr double kClassMargin = 2e-4;  // relative margin of the p > q test
constexpr int kPassBlock = 256;        // threads of a pass workgroup

// ---------------------------------------------------------------------------
// 2^(x/256) in fp64 for x <= 0 (a few ulp above 0 is fine; x must not be
// NaN).  The argument comes in 1/256ths of a power of two, so that rounding
// it to the nearest integer n is one add of the 1.5 * 2^52 shifter (its low
// word is n) and r = x - n is exact (both are multiples of the ulp of x and
// |r| <= 1/2).  2^(r/256) = exp(r ln2/256) by its degree-4 Taylor
// polynomial (the next term is below 4e-17); 2^(n mod 256 / 256) from a
// 256-entry table in LDS; then ldexp by n div 256.  A row's argument
// x = c z - M takes c = 256 log2(e)/T and M = c m, which are 256 times their
// values in base 2 exactly, so one fma forms it.

constexpr int kExpTab = 256;

struct ExpTable {
  double t[kExpTab];
};

// 2^(j/256), j = 0..255, correctly rounded to double.
__constant__ double kExp2Frac[256] = {
    0x1.0000000000000p+0  , 0x1.00b1afa5abcbfp+0  , 0x1.0163da9fb3335p+0  , 0x1.02168143b0281p+0,
    0x1.02c9a3e778061p+0  , 0x1.037d42e11bbccp+0  , 0x1.04315e86e7f85p+0  , 0x1.04e5f72f654b1p+0,
    0x1.059b0d3158574p+0  , 0x1.0650a0e3c1f89p+0  , 0x1.0706b29ddf6dep+0  , 0x1.07bd42b72a836p+0,
    0x1.0874518759bc8p+0  , 0x1.092bdf66607e0p+0  , 0x1.09e3ecac6f383p+0  , 0x1.0a9c79b1f3919p+0,
    0x1.0b5586cf9890fp+0  , 0x1.0c0f145e46c85p+0  , 0x1.0cc922b7247f7p+0  , 0x1.0d83b23395decp+0,
    0x1.0e3ec32d3d1a2p+0  , 0x1.0efa55fdfa9c5p+0  , 0x1.0fb66affed31bp+0  , 0x1.1073028d7233ep+0,
    0x1.11301d0125b51p+0  , 0x1.11edbab5e2ab6p+0  , 0x1.12abdc06c31ccp+0  , 0x1.136a814f204abp+0,
    0x1.1429aaea92de0p+0  , 0x1.14e95934f312ep+0  , 0x1.15a98c8a58e51p+0  , 0x1.166a45471c3c2p+0,
    0x1.172b83c7d517bp+0  , 0x1.17ed48695bbc0p+0  , 0x1.18af9388c8deap+0  , 0x1.1972658375d2fp+0,
    0x1.1a35beb6fcb75p+0  , 0x1.1af99f8138a1cp+0  , 0x1.1bbe084045cd4p+0  , 0x1.1c82f95281c6bp+0,
    0x1.1d4873168b9aap+0  , 0x1.1e0e75eb44027p+0  , 0x1.1ed5022fcd91dp+0  , 0x1.1f9c18438ce4dp+0,
    0x1.2063b88628cd6p+0  , 0x1.212be3578a819p+0  , 0x1.21f49917ddc96p+0  , 0x1.22bdda27912d1p+0,
    0x1.2387a6e756238p+0  , 0x1.2451ffb82140ap+0  , 0x1.251ce4fb2a63fp+0  , 0x1.25e85711ece75p+0,
    0x1.26b4565e27cddp+0  , 0x1.2780e341ddf29p+0  , 0x1.284dfe1f56381p+0  , 0x1.291ba7591bb70p+0,
    0x1.29e9df51fdee1p+0  , 0x1.2ab8a66d10f13p+0  , 0x1.2b87fd0dad990p+0  , 0x1.2c57e39771b2fp+0,
    0x1.2d285a6e4030bp+0  , 0x1.2df961f641589p+0  , 0x1.2ecafa93e2f56p+0  , 0x1.2f9d24abd886bp+0,
    0x1.306fe0a31b715p+0  , 0x1.31432edeeb2fdp+0  , 0x1.32170fc4cd831p+0  , 0x1.32eb83ba8ea32p+0,
    0x1.33c08b26416ffp+0  , 0x1.3496266e3fa2dp+0  , 0x1.356c55f929ff1p+0  , 0x1.36431a2de883bp+0,
    0x1.371a7373aa9cbp+0  , 0x1.37f26231e754ap+0  , 0x1.38cae6d05d866p+0  , 0x1.39a401b7140efp+0,
    0x1.3a7db34e59ff7p+0  , 0x1.3b57fbfec6cf4p+0  , 0x1.3c32dc313a8e5p+0  , 0x1.3d0e544ede173p+0,
    0x1.3dea64c123422p+0  , 0x1.3ec70df1c5175p+0  , 0x1.3fa4504ac801cp+0  , 0x1.40822c367a024p+0,
    0x1.4160a21f72e2ap+0  , 0x1.423fb2709468ap+0  , 0x1.431f5d950a897p+0  , 0x1.43ffa3f84b9d4p+0,
    0x1.44e086061892dp+0  , 0x1.45c2042a7d232p+0  , 0x1.46a41ed1d0057p+0  , 0x1.4786d668b3237p+0,
    0x1.486a2b5c13cd0p+0  , 0x1.494e1e192aed2p+0  , 0x1.4a32af0d7d3dep+0  , 0x1.4b17dea6db7d7p+0,
    0x1.4bfdad5362a27p+0  , 0x1.4ce41b817c114p+0  , 0x1.4dcb299fddd0dp+0  , 0x1.4eb2d81d8abffp+0,
    0x1.4f9b2769d2ca7p+0  , 0x1.508417f4531eep+0  , 0x1.516daa2cf6642p+0  , 0x1.5257de83f4eefp+0,
    0x1.5342b569d4f82p+0  , 0x1.542e2f4f6ad27p+0  , 0x1.551a4ca5d920fp+0  , 0x1.56070dde910d2p+0,
    0x1.56f4736b527dap+0  , 0x1.57e27dbe2c4cfp+0  , 0x1.58d12d497c7fdp+0  , 0x1.59c0827ff07ccp+0,
    0x1.5ab07dd485429p+0  , 0x1.5ba11fba87a03p+0  , 0x1.5c9268a5946b7p+0  , 0x1.5d84590998b93p+0,
    0x1.5e76f15ad2148p+0  , 0x1.5f6a320dceb71p+0  , 0x1.605e1b976dc09p+0  , 0x1.6152ae6cdf6f4p+0,
    0x1.6247eb03a5585p+0  , 0x1.633dd1d1929fdp+0  , 0x1.6434634ccc320p+0  , 0x1.652b9febc8fb7p+0,
    0x1.6623882552225p+0  , 0x1.671c1c70833f6p+0  , 0x1.68155d44ca973p+0  , 0x1.690f4b19e9538p+0,
    0x1.6a09e667f3bcdp+0  , 0x1.6b052fa75173ep+0  , 0x1.6c012750bdabfp+0  , 0x1.6cfdcddd47645p+0,
    0x1.6dfb23c651a2fp+0  , 0x1.6ef9298593ae5p+0  , 0x1.6ff7df9519484p+0  , 0x1.70f7466f42e87p+0,
    0x1.71f75e8ec5f74p+0  , 0x1.72f8286ead08ap+0  , 0x1.73f9a48a58174p+0  , 0x1.74fbd35d7cbfdp+0,
    0x1.75feb564267c9p+0  , 0x1.77024b1ab6e09p+0  , 0x1.780694fde5d3fp+0  , 0x1.790b938ac1cf6p+0,
    0x1.7a11473eb0187p+0  , 0x1.7b17b0976cfdbp+0  , 0x1.7c1ed0130c132p+0  , 0x1.7d26a62ff86f0p+0,
    0x1.7e2f336cf4e62p+0  , 0x1.7f3878491c491p+0  , 0x1.80427543e1a12p+0  , 0x1.814d2add106d9p+0,
    0x1.82589994cce13p+0  , 0x1.8364c1eb941f7p+0  , 0x1.8471a4623c7adp+0  , 0x1.857f4179f5b21p+0,
    0x1.868d99b4492edp+0  , 0x1.879cad931a436p+0  , 0x1.88ac7d98a6699p+0  , 0x1.89bd0a478580fp+0,
    0x1.8ace5422aa0dbp+0  , 0x1.8be05bad61778p+0  , 0x1.8cf3216b5448cp+0  , 0x1.8e06a5e0866d9p+0,
    0x1.8f1ae99157736p+0  , 0x1.902fed0282c8ap+0  , 0x1.9145b0b91ffc6p+0  , 0x1.925c353aa2fe2p+0,
    0x1.93737b0cdc5e5p+0  , 0x1.948b82b5f98e5p+0  , 0x1.95a44cbc8520fp+0  , 0x1.96bdd9a7670b3p+0,
    0x1.97d829fde4e50p+0  , 0x1.98f33e47a22a2p+0  , 0x1.9a0f170ca07bap+0  , 0x1.9b2bb4d53fe0dp+0,
    0x1.9c49182a3f090p+0  , 0x1.9d674194bb8d5p+0  , 0x1.9e86319e32323p+0  , 0x1.9fa5e8d07f29ep+0,
    0x1.a0c667b5de565p+0  , 0x1.a1e7aed8eb8bbp+0  , 0x1.a309bec4a2d33p+0  , 0x1.a42c980460ad8p+0,
    0x1.a5503b23e255dp+0  , 0x1.a674a8af46052p+0  , 0x1.a799e1330b358p+0  , 0x1.a8bfe53c12e59p+0,
    0x1.a9e6b5579fdbfp+0  , 0x1.ab0e521356ebap+0  , 0x1.ac36bbfd3f37ap+0  , 0x1.ad5ff3a3c2774p+0,
    0x1.ae89f995ad3adp+0  , 0x1.afb4ce622f2ffp+0  , 0x1.b0e07298db666p+0  , 0x1.b20ce6c9a8952p+0,
    0x1.b33a2b84f15fbp+0  , 0x1.b468415b749b1p+0  , 0x1.b59728de5593ap+0  , 0x1.b6c6e29f1c52ap+0,
    0x1.b7f76f2fb5e47p+0  , 0x1.b928cf22749e4p+0  , 0x1.ba5b030a1064ap+0  , 0x1.bb8e0b79a6f1fp+0,
    0x1.bcc1e904bc1d2p+0  , 0x1.bdf69c3f3a207p+0  , 0x1.bf2c25bd71e09p+0  , 0x1.c06286141b33dp+0,
    0x1.c199bdd85529cp+0  , 0x1.c2d1cd9fa652cp+0  , 0x1.c40ab5fffd07ap+0  , 0x1.c544778fafb22p+0,
    0x1.c67f12e57d14bp+0  , 0x1.c7ba88988c933p+0  , 0x1.c8f6d9406e7b5p+0  , 0x1.ca3405751c4dbp+0,
    0x1.cb720dcef9069p+0  , 0x1.ccb0f2e6d1675p+0  , 0x1.cdf0b555dc3fap+0  , 0x1.cf3155b5bab74p+0,
    0x1.d072d4a07897cp+0  , 0x1.d1b532b08c968p+0  , 0x1.d2f87080d89f2p+0  , 0x1.d43c8eacaa1d6p+0,
    0x1.d5818dcfba487p+0  , 0x1.d6c76e862e6d3p+0  , 0x1.d80e316c98398p+0  , 0x1.d955d71ff6075p+0,
    0x1.da9e603db3285p+0  , 0x1.dbe7cd63a8315p+0  , 0x1.dd321f301b460p+0  , 0x1.de7d5641c0658p+0,
    0x1.dfc97337b9b5fp+0  , 0x1.e11676b197d17p+0  , 0x1.e264614f5a129p+0  , 0x1.e3b333b16ee12p+0,
    0x1.e502ee78b3ff6p+0  , 0x1.e653924676d76p+0  , 0x1.e7a51fbc74c83p+0  , 0x1.e8f7977cdb740p+0,
    0x1.ea4afa2a490dap+0  , 0x1.eb9f4867cca6ep+0  , 0x1.ecf482d8e67f1p+0  , 0x1.ee4aaa2188510p+0,
    0x1.efa1bee615a27p+0  , 0x1.f0f9c1cb6412ap+0  , 0x1.f252b376bba97p+0  , 0x1.f3ac948dd7274p+0,
    0x1.f50765b6e4540p+0  , 0x1.f6632798844f8p+0  , 0x1.f7bfdad9cbe14p+0  , 0x1.f91d802243c89p+0,
    0x1.fa7c1819e90d8p+0  , 0x1.fbdba3692d514p+0  , 0x1.fd3c22b8f71f1p+0  , 0x1.fe9d96b2a23d9p+0,
};

template <int NT>
__device__ __forceinline__ void exp_table_init(ExpTable &tab) {
  for (int i = threadIdx.x; i < kExpTab; i += NT) tab.t[i] = kExp2Frac[i];
}

__device__ __forceinline__ double exp2_256(double x, const ExpTable &tab) {
  constexpr double kShift = 0x1.8p52;
  x = fmax(x, -281600.0);  // 2^-1100 is 0 in double; also maps -inf
  const double y = x + kShift;
  const double n = y - kShift;
  const int ni = (int)(uint32_t)__builtin_bit_cast(uint64_t, y);
  const double r = x - n;
  // (ln 2 / 256)^k / k!, correctly rounded
  double p = __builtin_fma(0x1.3b2ab6fba4e77p-39, r, 0x1.c6b08d704a0c0p-29);
  p = __builtin_fma(p, r, 0x1.ebfbdff82c58fp-19);
  p = __builtin_fma(p, r, 0x1.62e42fefa39efp-9);
  p = __builtin_fma(p, r, 1.0);
  return ldexp(tab.t[ni & 255] * p, ni >> 8);
}

constexpr double kLog2e256 = 0x1.71547652b82fep+8;  // 256 log2(e), log2(e) correctly rounded

// exponent scale of a row at temperature t: exp(z/t) = 2^(z c / 256)
__device__ __forceinline__ double exp2_scale(float t) { return kLog2e256 / (double)t; }

// a wave-uniform double moved to scalar registers
__device__ __forceinline__ double uniform_d(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------------------
// Workspace records of the draw.

struct DrawSeg {       // one (prefix, segment)
  double sp, sq;       // sums of w_p, w_q (residual: relative to the row max;
                       // p-row draw: relative to the segment max)
  double ap, aq;       // residual: sums of w_p, w_q over sure-positive tokens;
                       // p-row draw: ap = sum of w_p without the excluded token
  double ep, eq;       // residual: sums of w_p, w_q over margin tokens of equal logits
  float mseg;          // p-row draw: raw max logit of the segment
  int n_unc;           // stored uncertain tokens, -1 when the list overflowed
  int bad;             // p-row draw: a NaN logit in the segment
  int pad;
};

struct DrawUnc {       // one margin token, or one class of them (sums of its weights)
  double wp, wq;
  int v, pad;          // the token (the class's first token)
};

struct DrawMass {      // one (prefix, segment) in the pick
  double zr;           // residual mass (or p mass without the excluded token)
  double zp;           // p mass (fallback when the residual has no mass)
};

// P consecutive logits of a row, unit i (tokens [i*P, i*P + P)): a whole
// 16-byte vector, or a half or quarter of one (bf16).  kVec: 16-byte-aligned
// rows; otherwise P is 1.
template <typename E, bool kVec, int P>
__device__ __forceinline__ void load_unit(const typename E::elem *row, int i, float (&x)[P]) {
  if constexpr (!kVec) {
    static_assert(P == 1, "element-wise rows load one token at a time");
    x[0] = E::at(row, i);
  } else if constexpr (P == E::kPerVec) {
    E::unpack(reinterpret_cast<const vec16 *>(row)[i], x);
  } else if constexpr (sizeof(typename E::elem) == 2 && P == 4) {
    const uint2 a = reinterpret_cast<const uint2 *>(row)[i];
    x[0] = __uint_as_float(a.x << 16); x[1] = __uint_as_float(a.x & 0xffff0000u);
    x[2] = __uint_as_float(a.y << 16); x[3] = __uint_as_float(a.y & 0xffff0000u);
  } else if constexpr (sizeof(typename E::elem) == 2) {
    static_assert(P == 2, "unsupported unit");
    const uint32_t a = reinterpret_cast<const uint32_t *>(row)[i];
    x[0] = __uint_as_float(a << 16); x[1] = __uint_as_float(a & 0xffff0000u);
  } else {
    static_assert(P == 2, "unsupported unit");
    const float2 a = reinterpret_cast<const float2 *>(row)[i];
    x[0] = a.x;
    x[1] = a.y;
  }
}

// tokens per unit of the residual pass: four (fewer registers than a whole
// bf16 vector, so more waves)
template <typename E, bool kVec>
constexpr int pass_unit() {
  return kVec ? 4 : 1;
}

// The raw bits of one pass unit, so that the next unit's load can be in
// flight while the current one is computed: 8 bytes of bf16, 16 of fp32, or
// one element of a row without 16-byte alignment.
template <typename E, bool kVec>
struct PassRaw {
  static_assert(!kVec, "element-wise rows");
  using T = float;
  __device__ static T load(const typename E::elem *row, int i) { return E::at(row, i); }
  __device__ static void unpack(T t, float (&x)[1]) { x[0] = t; }
};
template <>
struct PassRaw<BF16, true> {
  using T = uint2;
  __device__ static T load(const BF16::elem *row, int i) {
    return reinterpret_cast<const uint2 *>(row)[i];
  }
  __device__ static void unpack(T a, float (&x)[4]) {
    x[0] = __uint_as_float(a.x << 16); x[1] = __uint_as_float(a.x & 0xffff0000u);
    x[2] = __uint_as_float(a.y << 16); x[3] = __uint_as_float(a.y & 0xffff0000u);
  }
};
template <>
struct PassRaw<F32, true> {
  using T = vec16;
  __device__ static T load(const F32::elem *row, int i) {
    return reinterpret_cast<const vec16 *>(row)[i];
  }
  __device__ static void unpack(T a, float (&x)[4]) { F32::unpack(a, x); }
};

// Visit the logits of [lo, hi) of one or two rows with NT threads, P tokens
// per unit: f(v, zp, zq).  kVec: rows start 16-byte aligned and hi - lo is a
// multiple of a vector.
// The next unit's load is issued before the current unit is visited.
template <typename E, bool kVec, bool kTwo, int NT, typename F>
__device__ __forceinline__ void visit_segment(const typename E::elem *rp, const typename E::elem *rq,
                                     int lo, int hi, F &&f) {
  constexpr int P = kVec ? E::kPerVec : 1;
  // raw bits of one unit: a 16-byte vector, or one element
  using T = typename std::conditional<kVec, vec16, float>::type;
  auto load = [](const typename E::elem *row, int i) -> T {
    if constexpr (kVec) return reinterpret_cast<const vec16 *>(row)[i];
    else return E::at(row, i);
  };
  auto unpack = [](const T &t, float (&x)[P]) {
    if constexpr (kVec) E::unpack(t, x);
    else x[0] = t;
  };
  const int iend = (hi + P - 1) / P;
  int i = lo / P + (int)threadIdx.x;
  T np_{}, nq_{};
  if (i < iend) {
    np_ = load(rp, i);
    if constexpr (kTwo) nq_ = load(rq, i);
  }
  for (; i < iend; i += NT) {
    const T cp_ = np_, cq_ = nq_;
    if (i + NT < iend) {
      np_ = load(rp, i + NT);
      if constexpr (kTwo) nq_ = load(rq, i + NT);
    }
    float xp[P], xq[P];
    unpack(cp_, xp);
    if constexpr (kTwo) unpack(cq_, xq);
#pragma unroll
    for (int e = 0; e < P; ++e) f(i * P + e, xp[e], kTwo ? xq[e] : 0.0f);
  }
}

// Sums of N doubles over the workgroup in a fixed order; valid in thread 0.
template <int NW, int N>
__device__ __forceinline__ void block_sums(double (&x)[N], double *lds /* N*NW */) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += __shfl_xor(x[i], off, 64);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int i = 0; i < N; ++i) lds[N * w + i] = x[i];
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll 1
    for (int k = 1; k < NW; ++k)
#pragma unroll
      for (int i = 0; i < N; ++i) x[i] += lds[N * k + i];
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// The pass: one workgroup per (prefix, segment), one record per segment.

template <int NT>
struct PassShared {
  ExpTable tab;
  double red[6 * (NT / 64)];
  float redf[NT / 64 + 1];
  int redi[NT / 64 + 1];
  int n_unc;
  DrawUnc unc[kUncList];
  double ukey[kUncList];  // the margin tokens' logit differences
  int uord[kUncList];
};

// One segment of a residual draw: the six sums of this thread in acc and the
// margin tokens in the workgroup's list.
template <typename E, bool kVec, int NT>
__device__ __forceinline__ void pass_residual(PassShared<NT> &S, const typename E::elem *rp,
                                              const typename E::elem *rq, int lo, int hi,
                                              double cp, double Mp, double cq, double Mq,
                                              double up, double dn, bool same_t,
                                              double (&acc)[6]) {
  // wave-uniform operands in scalar registers
  cp = uniform_d(cp);
  Mp = uniform_d(Mp);
  cq = uniform_d(cq);
  Mq = uniform_d(Mq);
  up = uniform_d(up);
  dn = uniform_d(dn);
  double sp = 0.0, sq = 0.0, ap = 0.0, aq = 0.0, ep = 0.0, eq = 0.0;
  // one unit of tokens at a time; its margin tokens are settled after it,
  // behind one branch.  The next unit's logits are loaded before the current
  // unit is computed, so a wave always has a load in flight.
  constexpr int P = pass_unit<E, kVec>();
  using Raw = PassRaw<E, kVec>;
  const int iend = (hi + P - 1) / P;
  int i = lo / P + (int)threadIdx.x;
  typename Raw::T np_ = {}, nq_ = {};
  if (i < iend) {
    np_ = Raw::load(rp, i);
    nq_ = Raw::load(rq, i);
  }
  for (; i < iend; i += NT) {
    const typename Raw::T cp_ = np_, cq_ = nq_;
    if (i + NT < iend) {
      np_ = Raw::load(rp, i + NT);
      nq_ = Raw::load(rq, i + NT);
    }
    float xp[P], xq[P];
    Raw::unpack(cp_, xp);
    Raw::unpack(cq_, xq);
    uint32_t margin = 0;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const double wp = exp2_256(__builtin_fma((double)xp[e], cp, -Mp), S.tab);
      const double wq = exp2_256(__builtin_fma((double)xq[e], cq, -Mq), S.tab);
      sp += wp;
      sq += wq;
      const bool pos = wp > up * wq;
      const double f = pos ? 1.0 : 0.0;
      ap = __builtin_fma(f, wp, ap);
      aq = __builtin_fma(f, wq, aq);
      margin |= (uint32_t)(!pos && wp > dn * wq) << e;
    }
    if (margin) {  // rare: the weights are recomputed (the same bits) rather than kept
#pragma unroll 1
      for (int e = 0; e < P; ++e) {
        if (!((margin >> e) & 1u)) continue;
        const double wp = exp2_256(__builtin_fma((double)xp[e], cp, -Mp), S.tab);
        const double wq = exp2_256(__builtin_fma((double)xq[e], cq, -Mq), S.tab);
        if (same_t && xp[e] == xq[e]) {
          ep += wp;
          eq += wq;
        } else {
          const int k = atomicAdd(&S.n_unc, 1);
          if (k < kUncList) {
            S.unc[k] = DrawUnc{wp, wq, i * P + e, 0};
            S.ukey[k] = (double)xp[e] - (double)xq[e];
          }
        }
      }
    }
  }
  acc[0] = sp;
  acc[1] = sq;
  acc[2] = ap;
  acc[3] = aq;
  acc[4] = ep;
  acc[5] = eq;
}

// The end of a segment: workgroup sums, the margin list (merged by class
// when longer than kUncCap) and the record.
template <int NT>
__device__ __forceinline__ void pass_finish(PassShared<NT> &S, double (&acc)[6], float mseg,
                                            int bad, bool classes, DrawSeg *__restrict__ segs,
                                            DrawUnc *__restrict__ uncs, int64_t so) {
  block_sums<NT / 64, 6>(acc, S.red);
  const int n = S.n_unc;
  int nout = -1;  // entries written; -1: the list overflowed
  if (n <= kUncCap) {
    // margin tokens in token order (distinct tokens: the ranks are a permutation)
    if ((int)threadIdx.x < n) {
      const DrawUnc e = S.unc[threadIdx.x];
      int rank = 0;
      for (int i = 0; i < n; ++i) rank += (S.unc[i].v < e.v);
      uncs[so * kUncCap + rank] = e;
    }
    nout = n;
  } else if (n <= kUncList && classes) {
    // merge by class: order by (difference, token), then each class's first
    // entry sums its class in that order
    for (int i = threadIdx.x; i < n; i += NT) {
      const double ki = S.ukey[i];
      const int vi = S.unc[i].v;
      int r = 0;
      for (int j = 0; j < n; ++j) r += (S.ukey[j] < ki) || (S.ukey[j] == ki && S.unc[j].v < vi);
      S.uord[r] = i;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < n; r += NT) {
      const int i = S.uord[r];
      if (r > 0 && S.ukey[S.uord[r - 1]] == S.ukey[i]) continue;  // not the first of its class
      int g = 0;
      for (int c = 1; c <= r; ++c) g += S.ukey[S.uord[c]] != S.ukey[S.uord[c - 1]];
      if (g >= kUncCap) continue;
      double swp = 0.0, swq = 0.0;
      for (int c = r; c < n && S.ukey[S.uord[c]] == S.ukey[i]; ++c) {
        swp += S.unc[S.uord[c]].wp;
        swq += S.unc[S.uord[c]].wq;
      }
      uncs[so * kUncCap + g] = DrawUnc{swp, swq, S.unc[i].v, 0};
    }
    int ng = 1;
    for (int c = 1; c < n; ++c) ng += S.ukey[S.uord[c]] != S.ukey[S.uord[c - 1]];
    nout = ng <= kUncCap ? ng : -1;
  }
  if (threadIdx.x == 0) {
    DrawSeg out{};
    out.sp = acc[0];
    out.sq = acc[1];
    out.ap = acc[2];
    out.aq = acc[3];
    out.ep = acc[4];
    out.eq = acc[5];
    out.mseg = mseg;
    out.bad = bad;
    out.n_unc = nout;
    segs[so] = out;
  }
}

template <typename E, bool kVec, int SEG>
__global__ __launch_bounds__(kPassBlock) __attribute__((amdgpu_waves_per_eu(6))) void kr_draw_pass(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q, int V,
    int nseg, float tp, float tq, const DrawDesc *__restrict__ desc,
    DrawSeg *__restrict__ segs, DrawUnc *__restrict__ uncs) {
  constexpr int NT = kPassBlock;
  __shared__ PassShared<NT> S;
  const int64_t b = blockIdx.x / nseg;
  const int seg = (int)(blockIdx.x - b * nseg);
  const DrawDesc d = desc[b];
  if (!d.valid) return;
  exp_table_init<NT>(S.tab);
  if (threadIdx.x == 0) S.n_unc = 0;
  __syncthreads();
  const typename E::elem *rp = p + d.prow * (int64_t)V;
  const double cp = exp2_scale(tp), cq = exp2_scale(tq);
  const int lo = seg * SEG, hi = min(V, lo + SEG);
  const int64_t so = b * nseg + seg;
  double acc[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  if (d.two) {
    const typename E::elem *rq = q + d.qrow * (int64_t)V;
    const double rho = (double)d.st.sp / (double)d.st.sq;  // fp32 estimate of S_p / S_q
    const double up = rho * (1.0 + kClassMargin), dn = rho * (1.0 - kClassMargin);
    pass_residual<E, kVec, NT>(S, rp, rq, lo, hi, cp, (double)d.st.mp * cp, cq,
                               (double)d.st.mq * cq, up, dn, tp == tq, acc);
    pass_finish<NT>(S, acc, kNegInf, 0, tp == tq, segs, uncs, so);
    return;
  }
  // p row: its max is known when it was scored (greedy rejection); a bonus
  // row takes this segment's max from a first sweep
  float mseg = d.st.mp;
  int bad = 0;
  if (!d.known) {
    float m = kNegInf;
    visit_segment<E, kVec, false, NT>(rp, rp, lo, hi, [&](int, float zp, float) {
      m = fmaxf(m, zp);
      bad |= (zp != zp);
    });
    mseg = block_max<NT / 64>(m, S.redf);
    bad = block_max_i<NT / 64>(bad, S.redi);
  }
  const double M = (double)fmaxf(mseg, kLowest) * cp;
  const int excl = d.excl;  // sp: every token; ap: all but the excluded one
  double sp = 0.0, ap = 0.0;
  visit_segment<E, kVec, false, NT>(rp, rp, lo, hi, [&](int v, float zp, float) {
    const double wp = exp2_256(__builtin_fma((double)zp, cp, -M), S.tab);
    sp += wp;
    ap = __builtin_fma(v != excl ? 1.0 : 0.0, wp, ap);
  });
  acc[0] = sp;
  acc[2] = ap;
  pass_finish<NT>(S, acc, mseg, bad, false, segs, uncs, so);
}

// Exact weights of the draw.
template <typename E>
struct DrawWeight {
  const typename E::elem *p, *q;
  double cp, cq, Mp, Mq, invSp, invSq;  // weight 2^((c z - M)/256) = exp((z - m)/T)
  bool resid;  // max(0, p - q); otherwise p with token excl zeroed
  int excl;
  // weight of token v from its two logits
  __device__ __forceinline__ double from(int v, float zp, float zq, const ExpTable &tab) const {
    const double pv = exp2_256(__builtin_fma((double)zp, cp, -Mp), tab) * invSp;
    if (!resid) return v == excl ? 0.0 : pv;
    const double qv = exp2_256(__builtin_fma((double)zq, cq, -Mq), tab) * invSq;
    const double dd = pv - qv;
    return dd > 0.0 ? dd : 0.0;
  }
};

// Fixed-order reductions over the 64 lanes of a wave (an xor butterfly:
// every lane ends with the same bits).
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Exact row normalisers of the draw from the pass's segment sums; every wave
// computes them (lane l adds segments l, l + 64, ..., then the lanes are
// summed).  Returns false for an invalid bonus row.
template <typename E>
__device__ __forceinline__ bool draw_setup(const typename E::elem *rp,
                                           const typename E::elem *rq, const DrawDesc &d,
                                           const DrawSeg *S, int nseg, float tp, float tq,
                                           DrawWeight<E> &W) {
  const int lane = threadIdx.x & 63;
  W.p = rp;
  W.q = rq;
  W.cp = exp2_scale(tp);
  W.cq = exp2_scale(tq);
  W.resid = d.two != 0;
  W.excl = d.excl;
  double Sp = 0.0, Sq = 1.0;
  // segment sums relative to one max (residual rows and scored p rows) or to
  // their segments' maxima (bonus rows)
  if (W.resid) {
    W.Mp = (double)d.st.mp * W.cp;
    W.Mq = (double)d.st.mq * W.cq;
    double a = 0.0, c = 0.0;
    for (int s = lane; s < nseg; s += 64) {
      a += S[s].sp;
      c += S[s].sq;
    }
    Sp = wave_sum_d(a);
    Sq = wave_sum_d(c);
  } else {
    float m = kNegInf;
    int bad = 0;
    for (int s = lane; s < nseg; s += 64) {
      m = fmaxf(m, S[s].mseg);
      bad |= S[s].bad;
    }
    const float mr = wave_max_f(m);
    if (__any(bad) || mr == kNegInf || mr == -kNegInf) return false;
    W.Mp = (double)mr * W.cp;
    W.Mq = 0.0;
    double a = 0.0;
    for (int s = lane; s < nseg; s += 64) {
      const double Ms = (double)fmaxf(S[s].mseg, kLowest) * W.cp;
      a += (S[s].mseg == mr) ? S[s].sp : S[s].sp * exp2((Ms - W.Mp) * 0x1.0p-8);
    }
    Sp = wave_sum_d(a);
  }
  W.invSp = 1.0 / Sp;
  W.invSq = 1.0 / Sq;
  return true;
}

// The weights of the kRun consecutive tokens from a of a segment ending at hi.
template <typename E, bool kVec, int kRun>
__device__ __forceinline__ void run_weights(const DrawWeight<E> &W, int a, int hi,
                                            const ExpTable &tab, double (&w)[kRun]) {
  if constexpr (kVec) {
    constexpr int P = E::kPerVec;
    static_assert(kRun % P == 0, "a run is whole 16-byte vectors");
    const vec16 *vp = reinterpret_cast<const vec16 *>(W.p + a);
    const vec16 *vq = reinterpret_cast<const vec16 *>(W.q + (W.resid ? a : 0));
#pragma unroll
    for (int c = 0; c < kRun / P; ++c) {
      float xp[P], xq[P];
      const bool in = a + c * P < hi;  // hi - lo is a multiple of P on this path
      if (in) {
        E::unpack(vp[c], xp);
        if (W.resid) E::unpack(vq[c], xq);
      }
#pragma unroll
      for (int e = 0; e < P; ++e)
        w[c * P + e] = in ? W.from(a + c * P + e, xp[e], W.resid ? xq[e] : 0.0f, tab) : 0.0;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      const int v = a + i;
      w[i] = (v < hi) ? W.from(v, E::at(W.p, v), W.resid ? E::at(W.q, v) : 0.0f, tab) : 0.0;
    }
  }
}

// Exact residual mass of one segment (all NT threads); valid in thread 0.
template <typename E, bool kVec, int NT, int SEG>
__device__ __forceinline__ double segment_mass_exact(const DrawWeight<E> &W, int V, int seg,
                                                     const ExpTable &tab, double *ldsd) {
  const int lo = seg * SEG, hi = min(V, lo + SEG);
  double z = 0.0;
  visit_segment<E, kVec, true, NT>(W.p, W.q, lo, hi, [&](int v, float zp, float zq) {
    z += W.from(v, zp, zq, tab);
  });
  return block_sum_d<NT / 64>(z, ldsd);
}

// Exclusive prefix sum over the workgroup in thread order (fixed pattern).
template <int NW>
__device__ __forceinline__ double block_exclusive_scan(double x, double *lds /* NW */) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(inc, off, 64);
    if (lane >= off) inc += y;
  }
  if (lane == 63) lds[w] = inc;
  __syncthreads();
  double base = 0.0;
#pragma unroll 1
  for (int i = 0; i < w; ++i) base += lds[i];
  const double prev = __shfl_up(inc, 1, 64);
  __syncthreads();
  return base + (lane == 0 ? 0.0 : prev);
}

// The pick: one workgroup of kPickBlock threads per prefix.  mass is global
// scratch for the segment masses of vocabularies with more than kPickSegs
// segments.
template <typename E, bool kVec, int SEG>
__global__ __launch_bounds__(kPickBlock) void kr_draw_pick(
    const typename E::elem *__restrict__ p, const typename E::elem *__restrict__ q, int V,
    int nseg, float tp, float tq, uint64_t seed, uint64_t row_base,
    const DrawDesc *__restrict__ desc, const DrawSeg *__restrict__ segs,
    const DrawUnc *__restrict__ uncs, DrawMass *__restrict__ mass,
    int32_t *__restrict__ selected, int32_t *__restrict__ accept_len,
    int32_t *__restrict__ next_token) {
  constexpr int NT = kPickBlock, NW = NT / 64;
  // tokens per thread in the scan of one segment (whole 16-byte vectors); in a
  // segment shorter than NT * kRun the threads past its end hold no tokens
  constexpr int kRun = SEG / NT > 8 ? SEG / NT : 8;
  __shared__ ExpTable tab;
  __shared__ double ldsd[NW + 1];
  __shared__ int ldsi[NW + 1];
  __shared__ DrawSeg segl[kPickSegs];  // the prefix's records, when they fit
  __shared__ DrawMass massl[kPickSegs];
  __shared__ DrawUnc uncl[kPickUncSegs * kUncCap];
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  // the records are staged together with the descriptor's load (a prefix
  // without a draw has stale records, which it never reads)
  const bool staged = nseg <= kPickSegs;
  const bool unc_staged = nseg <= kPickUncSegs;
  if (staged)
    for (int s = tid; s < nseg; s += NT) segl[s] = segs[b * nseg + s];
  if (unc_staged)  // every slot: the lists' lengths are not known yet
    for (int i = tid; i < nseg * kUncCap; i += NT) uncl[i] = uncs[b * nseg * kUncCap + i];
  const DrawDesc d = desc[b];
  exp_table_init<NT>(tab);
  __syncthreads();
  if (!d.valid) return;
  const DrawSeg *S = staged ? segl : segs + b * nseg;
  const DrawUnc *U = unc_staged ? uncl : uncs + b * nseg * kUncCap;
  DrawMass *ms = staged ? massl : mass + b * nseg;
  const typename E::elem *rp = p + d.prow * (int64_t)V;
  const typename E::elem *rq = d.two ? q + d.qrow * (int64_t)V : nullptr;
  const bool residual = d.two != 0;
  DrawWeight<E> W;
  if (!draw_setup<E>(rp, rq, d, S, nseg, tp, tq, W)) {
    if (tid == 0) {  // invalid bonus row (the scored rows were checked earlier)
      if (selected) selected[b] = -1;
      accept_len[b] = -1;
      next_token[b] = -1;
    }
    return;
  }

  // per-segment masses (the exactly recomputed residual segments just below)
  for (int s = tid; s < nseg; s += NT) {
    const DrawSeg g = S[s];
    DrawMass m{};
    if (residual) {
      m.zp = g.sp * W.invSp;
      if (g.n_unc >= 0) {
        double z = g.ap * W.invSp - g.aq * W.invSq;
        const double ze = g.ep * W.invSp - g.eq * W.invSq;  // the class of equal logits
        if (ze > 0.0) z += ze;
        const DrawUnc *u = U + (int64_t)s * kUncCap;
        for (int i = 0; i < g.n_unc; ++i) {
          const DrawUnc e = u[i];
          const double dd = e.wp * W.invSp - e.wq * W.invSq;
          if (dd > 0.0) z += dd;
        }
        m.zr = z;
      }
    } else {  // p row: zp with every token, zr without the excluded one
      const double Ms = (double)fmaxf(g.mseg, kLowest) * W.cp;
      const double scale = (g.mseg == kNegInf) ? 0.0 : exp2((Ms - W.Mp) * 0x1.0p-8);
      m.zp = g.sp * scale * W.invSp;
      m.zr = g.ap * scale * W.invSp;
    }
    ms[s] = m;
  }
  __syncthreads();
  int overflow = 0;
  for (int s = lane; s < nseg; s += 64) overflow |= residual && S[s].n_unc < 0;
  if (__any(overflow)) {  // segments whose list overflowed: exact, all threads
    for (int s = 0; s < nseg; ++s) {
      if (S[s].n_unc >= 0) continue;
      const double z = segment_mass_exact<E, kVec, NT, SEG>(W, V, s, tab, ldsd);
      if (tid == 0) ms[s].zr = z;
      __syncthreads();
    }
  }

  double zl = 0.0;
  for (int s = lane; s < nseg; s += 64) zl += ms[s].zr;
  const double zr = wave_sum_d(zl);
  const bool use_r = zr > 0.0;  // a residual without mass draws from p
  W.resid = residual && use_r;
  if (!use_r) W.excl = -1;
  double Z = zr;
  if (!use_r) {
    zl = 0.0;
    for (int s = lane; s < nseg; s += 64) zl += ms[s].zp;
    Z = wave_sum_d(zl);
  }
  const double t = counter_uniform(seed, row_base + (uint64_t)b, (uint64_t)d.pos,
                                   (uint64_t)d.purpose) * Z;

  // the segment that holds t: the first whose inclusive prefix sum of masses
  // exceeds it (a scan over lanes, or a serial one past 64 segments)
  double cum = 0.0;
  int s0 = -1;
  if (nseg <= 64) {
    const double w = lane < nseg ? (use_r ? ms[lane].zr : ms[lane].zp) : 0.0;
    double incl = w;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const double excl = __shfl_up(incl, 1, 64);
    const uint64_t hit = __ballot(lane < nseg && incl > t);
    if (hit) {
      s0 = __ffsll((unsigned long long)hit) - 1;
      cum = __shfl(lane == 0 ? 0.0 : excl, s0, 64);
    }
  } else {
    // lane l holds the run of segments [l c, l c + c); the first lane whose
    // inclusive sum exceeds t names the run, and a walk from the run's start
    // finds the segment (it goes on past the run if rounding moved the hit)
    const int c = (nseg + 63) >> 6;
    const int r0 = lane * c, r1 = min(nseg, r0 + c);
    double w = 0.0;
    for (int s = r0; s < r1; ++s) w += use_r ? ms[s].zr : ms[s].zp;
    double incl = w;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const double excl = __shfl_up(incl, 1, 64);
    const uint64_t hit = __ballot(r0 < nseg && incl > t);
    if (hit) {
      const int l0 = __ffsll((unsigned long long)hit) - 1;
      cum = __shfl(lane == 0 ? 0.0 : excl, l0, 64);
      for (int s = l0 * c; s < nseg; ++s) {
        const double ws = use_r ? ms[s].zr : ms[s].zp;
        if (cum + ws > t) {
          s0 = s;
          break;
        }
        cum += ws;
      }
    }
  }
  int tok = -1;
  if (s0 >= 0) {
    for (int s = s0; s < nseg; ++s) {
      // thread tid owns tokens [a, a + kRun) of the segment, kept in registers
      const int hi = min(V, (s + 1) * SEG);
      const int a = s * SEG + tid * kRun;
      double w[kRun];
      run_weights<E, kVec, kRun>(W, a, hi, tab, w);
      double loc = 0.0;
#pragma unroll
      for (int i = 0; i < kRun; ++i) loc += w[i];
      double C = cum + block_exclusive_scan<NW>(loc, ldsd);
      int found = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kRun; ++i) {
        C += w[i];
        if (found == 0x7fffffff && w[i] > 0.0 && C > t) found = a + i;
      }
      found = block_min_i<NW>(found, ldsi);
      if (found != 0x7fffffff) {
        tok = found;
        break;
      }
      cum += use_r ? ms[s].zr : ms[s].zp;
    }
  }
  // t at or past the total through rounding: the last token with weight
  for (int s = nseg - 1; s >= 0 && tok < 0; --s) {
    const int hi = min(V, (s + 1) * SEG);
    const int a = s * SEG + tid * kRun;
    double w[kRun];
    run_weights<E, kVec, kRun>(W, a, hi, tab, w);
    int last = -1;
#pragma unroll
    for (int i = 0; i < kRun; ++i)
      if (w[i] > 0.0) last = a + i;
    tok = block_max_i<NW>(last, ldsi);
  }
  if (tid == 0) next_token[b] = tok;
}

}  // namespace svd
