// kr_adl.hpp -- adaptive draft length: each sequence's next window.
//
// DiffuSpec section 4.3 ("Adaptive Draft Length"): the controller sets the
// next draft length from the EOS-aware generated length and the accepted
// length, growing it while acceptance keeps pace with generation on average
// and holding it once the generated length saturates at EOS; shrinking toward
// the recent accepted streak when acceptance lags keeps a sequence from
// over-drafting (DiffuSpec section 6).  The recent lengths are averages in
// 1/256ths of a token, moved by 2^-shift of the gap and rounded down, so every
// decision is an exact integer comparison.
#pragma once

#include "svd_device.hpp"

namespace svd {

constexpr int32_t kAdlStateMax = 1 << 20;  // 256 * the largest window

// One thread per prefix.  avg [B][2] = {accepted, generated} in 1/256ths of a
// token (in/out); next [B] = the next window, -1 for a window or state out of
// range, this window again when the prefix's outputs were -1.
__global__ __launch_bounds__(kBlock) void kr_adl(
    const int32_t *__restrict__ drafts, const int32_t *__restrict__ selected,
    const int32_t *__restrict__ accept_len, const int32_t *__restrict__ gamma_b, int eos,
    int64_t B, int K, int gamma, int k_min, int k_max, int step, int shift, int slack,
    int32_t *__restrict__ avg, int32_t *__restrict__ next) {
  const int64_t b = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (b >= B) return;
  const int n = gamma_b ? gamma_b[b] : gamma;
  if (n < 1 || n > gamma) {
    next[b] = -1;
    return;
  }
  const int k = selected[b], L = accept_len[b];
  if (k < 0 || k >= K || L < 0 || L > n) {
    next[b] = n;
    return;
  }
  int A = avg[2 * b], G = avg[2 * b + 1];
  if (A < 0 || A > kAdlStateMax || G < 0 || G > kAdlStateMax) {
    next[b] = -1;
    return;
  }
  // generated length of the kept draft: through its first EOS, or the window
  int g = n;
  if (eos >= 0) {
    const int32_t *row = drafts + ((int64_t)b * K + k) * gamma;
    for (int j = 0; j < n; ++j)
      if (row[j] == eos) {
        g = j + 1;
        break;
      }
  }
  // an arithmetic right shift divides by 2^shift rounding toward -infinity
  A += (256 * L - A) >> shift;
  G += (256 * g - G) >> shift;
  avg[2 * b] = A;
  avg[2 * b + 1] = G;
  int w;
  if (g < n)
    w = n;  // the draft ended at EOS inside the window: hold
  else if (A + slack >= G)
    w = n + step;  // acceptance keeps pace with generation: expand
  else
    w = min(n, ((A + 255) >> 8) + 1);  // acceptance lags: the recent streak plus one
  next[b] = max(k_min, min(k_max, w));
}

}  // namespace svd
