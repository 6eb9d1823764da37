// svd_api.hip -- the C ABI declared in include/svd.h: argument checks,
// workspace layout and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <tuple>
#include <utility>

#include "svd.h"
#include "kr_beta.hpp"
#include "kr_draw.hpp"
#include "kr_fused.hpp"
#include "kr_rowstats.hpp"
#include "kr_select.hpp"

namespace {

using namespace svd;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// SVD_FUSED selects the one-launch path (kr_fused); 0 builds the chain of
// separate kernels instead, for comparison.
#ifndef SVD_FUSED
#define SVD_FUSED 0
#endif

struct Layout {
  size_t stats, alpha, desc, segs, uncs, mass, sync, total;
  int nseg;
  int64_t nsync;
};

bool sizes_ok(int64_t B, int32_t K, int32_t G, int32_t V) {
  if (B < 1 || K < 1 || G < 1 || V < 1) return false;
  if (K > SVD_MAX_K || G > SVD_MAX_GAMMA) return false;
  const int64_t nseg = ((int64_t)V + kDrawSeg - 1) / kDrawSeg;
  const int64_t lim = (int64_t)1 << 31;
  if (B >= lim / ((int64_t)K * G)) return false;  // B*K*gamma workgroups
  if (B >= lim / nseg) return false;              // B*nseg workgroups
  if (B * ((int64_t)K * G + nseg) >= lim) return false;  // workgroups of the fused launch
  return true;
}

Layout layout(int64_t B, int32_t K, int32_t G, int32_t V) {
  Layout L{};
  const size_t rp = (size_t)B * K * G;
  L.nseg = (int)(((int64_t)V + kDrawSeg - 1) / kDrawSeg);
  size_t off = 0;
  L.stats = off;
  off = align_up(off + rp * sizeof(RowStats));
  L.alpha = off;
  off = align_up(off + rp * sizeof(float));
  L.desc = off;
  off = align_up(off + (size_t)B * sizeof(DrawDesc));
  L.segs = off;
  off = align_up(off + (size_t)B * L.nseg * sizeof(DrawSeg));
  L.uncs = off;
  off = align_up(off + (size_t)B * L.nseg * kUncCap * sizeof(DrawUnc));
  L.mass = off;
  off = align_up(off + (size_t)B * L.nseg * sizeof(DrawMass));
  L.sync = off;
  L.nsync = 2 + 3 * B;
  off = align_up(off + (size_t)L.nsync * sizeof(unsigned));
  L.total = off;
  return L;
}

// Launch through hipLaunchKernel so that the launch status comes back
// directly (no reliance on the thread's sticky last-error state).
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                  Args &&...args) {
  std::tuple<KArgs...> vals(std::forward<Args>(args)...);
  void *ptrs[sizeof...(KArgs) ? sizeof...(KArgs) : 1];
  std::apply([&](auto &...v) {
    int i = 0;
    ((ptrs[i++] = (void *)&v), ...);
  }, vals);
  return hipLaunchKernel((const void *)kernel, grid, block, ptrs, 0, stream);
}

// ---------------------------------------------------------------------------
// Kernel timing (svd_profile_*): events around every launch of a call.

constexpr int kProfCalls = 4096;
constexpr int kProfMarks = SVD_KERNEL_COUNT + 1;

struct Profiler {
  bool on = false;
  int ncalls = 0;
  bool created[kProfCalls] = {};
  hipEvent_t ev[kProfCalls][kProfMarks];
  int kid[kProfCalls][kProfMarks];
  int nmarks[kProfCalls] = {};
};
Profiler g_prof;

struct CallTimer {
  int slot = -1;
  hipStream_t stream;
  explicit CallTimer(hipStream_t s) : stream(s) {
    if (!g_prof.on || g_prof.ncalls >= kProfCalls) return;
    slot = g_prof.ncalls++;
    if (!g_prof.created[slot]) {
      for (int i = 0; i < kProfMarks; ++i)
        if (hipEventCreate(&g_prof.ev[slot][i]) != hipSuccess) {
          slot = -1;
          g_prof.ncalls--;
          return;
        }
      g_prof.created[slot] = true;
    }
    g_prof.nmarks[slot] = 0;
  }
  // mark the start of kernel `kernel_id` (or the end of the call with -1)
  void mark(int kernel_id) {
    if (slot < 0) return;
    int &n = g_prof.nmarks[slot];
    if (n >= kProfMarks) return;
    if (hipEventRecord(g_prof.ev[slot][n], stream) != hipSuccess) return;
    g_prof.kid[slot][n] = kernel_id;
    ++n;
  }
};

#define SVD_LAUNCH(...)                               \
  do {                                                \
    if (launch(__VA_ARGS__) != hipSuccess) return SVD_EHIP; \
  } while (0)

template <typename E, bool kVec>
int run(const void *p_logits, const void *q_logits, const int32_t *drafts, int64_t B, int32_t K,
        int32_t G, int32_t V, float tp, float tq, uint64_t seed, uint64_t row_base,
        int32_t *selected, int32_t *accept_len, int32_t *next_token, float *scores, float *alpha,
        float *beta, void *workspace, hipStream_t stream) {
  using T = typename E::elem;
  const T *p = static_cast<const T *>(p_logits);
  const T *q = static_cast<const T *>(q_logits);
  const Layout Lo = layout(B, K, G, V);
  char *ws = static_cast<char *>(workspace);
  RowStats *stats = reinterpret_cast<RowStats *>(ws + Lo.stats);
  float *alpha_ws = reinterpret_cast<float *>(ws + Lo.alpha);
  DrawDesc *desc = reinterpret_cast<DrawDesc *>(ws + Lo.desc);
  DrawSeg *segs = reinterpret_cast<DrawSeg *>(ws + Lo.segs);
  DrawUnc *uncs = reinterpret_cast<DrawUnc *>(ws + Lo.uncs);
  DrawMass *mass = reinterpret_cast<DrawMass *>(ws + Lo.mass);
  const unsigned rp = (unsigned)((int64_t)B * K * G);
  const unsigned nb = (unsigned)B;
  const unsigned nbs = (unsigned)(B * Lo.nseg);
  // log2(e) / T folded into one factor per row: exp(z/T) = exp2(z * c)
  const float cp = (float)(1.4426950408889634 / (double)tp);
  const float cq = (float)(1.4426950408889634 / (double)tq);

  CallTimer tm(stream);
  if (SVD_FUSED) {
    // lag of the fused schedule: about one generation of resident workgroups
    static int blocks_per_cu = [] {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kr_fused<E, kVec>, kFusedBlock, 0) !=
              hipSuccess ||
          n < 1)
        n = 1;
      return n;
    }();
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    const int64_t P = (int64_t)K * G;
#ifndef SVD_LAG_MUL
#define SVD_LAG_MUL 1
#endif
    // SVD_LAG_MUL scales the lag; 0 streams every row pair before any draw
    const int64_t lag = SVD_LAG_MUL == 0 ? B : SVD_LAG_MUL * (((int64_t)cus * blocks_per_cu + P - 1) / P);
    FusedArgs<E> fa;
    fa.p = p;
    fa.q = q;
    fa.drafts = drafts;
    fa.B = B;
    fa.K = K;
    fa.gamma = G;
    fa.V = V;
    fa.nseg = Lo.nseg;
    fa.lag = (int)(lag < 1 ? 1 : (lag > B ? B : lag));
    fa.tp = tp;
    fa.tq = tq;
    fa.cp = cp;
    fa.cq = cq;
    fa.seed = seed;
    fa.row_base = row_base;
    fa.selected = selected;
    fa.accept_len = accept_len;
    fa.next_token = next_token;
    fa.scores = scores;
    fa.alpha_out = alpha;
    fa.stats = stats;
    fa.alpha_ws = alpha_ws;
    fa.desc = desc;
    fa.segs = segs;
    fa.uncs = uncs;
    fa.mass = mass;
    fa.sync = reinterpret_cast<unsigned *>(ws + Lo.sync);
    const int64_t nsync = Lo.nsync;
    const unsigned init_grid = (unsigned)std::min<int64_t>((nsync + 255) / 256, 1024);
    tm.mark(SVD_KERNEL_INIT);
    SVD_LAUNCH(kr_fused_init, dim3(init_grid), dim3(256), stream, fa.sync, nsync);
    tm.mark(SVD_KERNEL_FUSED);
    const unsigned items = (unsigned)(B * (P + (Lo.nseg + kDrawGroup - 1) / kDrawGroup));
    SVD_LAUNCH(kr_fused<E, kVec>, dim3(items), dim3(kFusedBlock), stream, fa);
    if (beta) {
      tm.mark(SVD_KERNEL_BETA);
      SVD_LAUNCH(kr_beta<E, kVec>, dim3(rp), dim3(kBlock), stream, p, q, G, V, cp, cq,
                 (const RowStats *)stats, beta);
    }
    tm.mark(-1);
    return SVD_OK;
  }
  tm.mark(SVD_KERNEL_ROWSTATS);
  SVD_LAUNCH(kr_rowstats<E, kVec>, dim3(rp), dim3(kRowBlock), stream, p, q, drafts, G, V, cp, cq,
             stats, alpha_ws, alpha);
  if (beta) {
    tm.mark(SVD_KERNEL_BETA);
    SVD_LAUNCH(kr_beta<E, kVec>, dim3(rp), dim3(kBlock), stream, p, q, G, V, cp, cq,
               (const RowStats *)stats, beta);
  }
  tm.mark(SVD_KERNEL_SELECT);
  SVD_LAUNCH(kr_select, dim3(nb), dim3(64), stream, (const float *)alpha_ws, K, G, seed,
             row_base, selected, accept_len, next_token, scores, desc);
  tm.mark(SVD_KERNEL_DRAW_PASS);
  SVD_LAUNCH(kr_draw_pass<E, kVec>, dim3(nbs), dim3(kBlock), stream, p, q, K, G, V, Lo.nseg, tp,
             tq, (const RowStats *)stats, (const DrawDesc *)desc, segs, uncs);
  tm.mark(SVD_KERNEL_DRAW_FIX);
  SVD_LAUNCH(kr_draw_fix<E, kVec>, dim3(nbs), dim3(kBlock), stream, p, q, K, G, V, Lo.nseg, tp,
             tq, (const RowStats *)stats, (const DrawDesc *)desc, (const DrawSeg *)segs, mass);
  tm.mark(SVD_KERNEL_DRAW_PICK);
  SVD_LAUNCH(kr_draw_pick<E, kVec>, dim3(nb), dim3(kBlock), stream, p, q, K, G, V, Lo.nseg, tp,
             tq, seed, row_base, (const RowStats *)stats, (const DrawDesc *)desc,
             (const DrawSeg *)segs, (const DrawUnc *)uncs, mass, selected, accept_len,
             next_token);
  tm.mark(-1);
  return SVD_OK;
}

bool temp_ok(float t) { return std::isfinite(t) && t > 0.0f; }

int dispatch(const void *p, const void *q, const int32_t *drafts, svd_dtype_t dtype, int64_t B,
             int32_t K, int32_t G, int32_t V, float tp, float tq, uint64_t seed,
             uint64_t row_base, int32_t *selected, int32_t *accept_len, int32_t *next_token,
             float *scores, float *alpha, float *beta, void *workspace, size_t workspace_bytes,
             void *hip_stream) {
  if (!p || !q || !drafts || !accept_len || !next_token || !workspace) return SVD_EINVAL;
  if (dtype != SVD_F32 && dtype != SVD_BF16) return SVD_EDTYPE;
  if (!sizes_ok(B, K, G, V) || !temp_ok(tp) || !temp_ok(tq)) return SVD_EINVAL;
  if (((uintptr_t)workspace) % kAlign != 0) return SVD_EINVAL;
  if (workspace_bytes < layout(B, K, G, V).total) return SVD_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const size_t es = dtype == SVD_F32 ? 4 : 2;
  // 16-byte loads need every row to start 16-byte aligned
  const bool vec = ((size_t)V * es) % 16 == 0 && ((uintptr_t)p) % 16 == 0 &&
                   ((uintptr_t)q) % 16 == 0;
  if (dtype == SVD_BF16) {
    return vec ? run<BF16, true>(p, q, drafts, B, K, G, V, tp, tq, seed, row_base, selected,
                                 accept_len, next_token, scores, alpha, beta, workspace, s)
               : run<BF16, false>(p, q, drafts, B, K, G, V, tp, tq, seed, row_base, selected,
                                  accept_len, next_token, scores, alpha, beta, workspace, s);
  }
  return vec ? run<F32, true>(p, q, drafts, B, K, G, V, tp, tq, seed, row_base, selected,
                              accept_len, next_token, scores, alpha, beta, workspace, s)
             : run<F32, false>(p, q, drafts, B, K, G, V, tp, tq, seed, row_base, selected,
                               accept_len, next_token, scores, alpha, beta, workspace, s);
}

}  // namespace

extern "C" {

size_t svd_workspace_bytes(int64_t B, int32_t K, int32_t gamma, int32_t V) {
  if (!sizes_ok(B, K, gamma, V)) return 0;
  return layout(B, K, gamma, V).total;
}

int svd_verify(const void *p_logits, const void *q_logits, const int32_t *draft,
               svd_dtype_t dtype, int64_t B, int32_t gamma, int32_t V, float temp_p,
               float temp_q, uint64_t seed, uint64_t row_base, int32_t *accept_len,
               int32_t *next_token, float *alpha, float *beta, void *workspace,
               size_t workspace_bytes, void *hip_stream) {
  return dispatch(p_logits, q_logits, draft, dtype, B, 1, gamma, V, temp_p, temp_q, seed,
                  row_base, nullptr, accept_len, next_token, nullptr, alpha, beta, workspace,
                  workspace_bytes, hip_stream);
}

int svd_select_and_verify(const void *p_logits, const void *q_logits, const int32_t *drafts,
                          svd_dtype_t dtype, int64_t B, int32_t K, int32_t gamma, int32_t V,
                          float temp_p, float temp_q, uint64_t seed, uint64_t row_base,
                          int32_t *selected, int32_t *accept_len, int32_t *next_token,
                          float *scores, float *alpha, float *beta, void *workspace,
                          size_t workspace_bytes, void *hip_stream) {
  if (!selected) return SVD_EINVAL;
  return dispatch(p_logits, q_logits, drafts, dtype, B, K, gamma, V, temp_p, temp_q, seed,
                  row_base, selected, accept_len, next_token, scores, alpha, beta, workspace,
                  workspace_bytes, hip_stream);
}

const char *svd_strerror(int status) {
  switch (status) {
    case SVD_OK: return "success";
    case SVD_EINVAL: return "invalid argument (null pointer, size out of range, bad temperature or misaligned workspace)";
    case SVD_EDTYPE: return "unsupported logit dtype";
    case SVD_EWORKSPACE: return "workspace smaller than svd_workspace_bytes()";
    case SVD_EHIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int svd_profile_enable(int on) {
  g_prof.on = on != 0;
  return SVD_OK;
}

int svd_profile_read(double *ms, int64_t *launches, int n) {
  if (!ms || n < 0) return SVD_EINVAL;
  for (int i = 0; i < n; ++i) {
    ms[i] = 0.0;
    if (launches) launches[i] = 0;
  }
  for (int c = 0; c < g_prof.ncalls; ++c) {
    const int nm = g_prof.nmarks[c];
    if (nm == 0) continue;
    if (hipEventSynchronize(g_prof.ev[c][nm - 1]) != hipSuccess) return SVD_EHIP;
    for (int i = 0; i + 1 < nm; ++i) {
      const int k = g_prof.kid[c][i];
      if (k < 0 || k >= n) continue;
      float t = 0.0f;
      if (hipEventElapsedTime(&t, g_prof.ev[c][i], g_prof.ev[c][i + 1]) != hipSuccess)
        return SVD_EHIP;
      ms[k] += t;
      if (launches) launches[k] += 1;
    }
  }
  g_prof.ncalls = 0;
  return SVD_OK;
}

}  // extern "C"
