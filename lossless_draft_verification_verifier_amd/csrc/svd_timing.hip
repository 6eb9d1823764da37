// svd_timing.hip -- the timing build's event records (svd_timing.h).  Linked
// only into libsvd_timed.so; the product library has no part of it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "svd.h"
#include "svd_timing.h"
#include "svd_timing.hpp"

namespace {

constexpr int kProfCalls = 4096;
constexpr int kProfLaunches = 48;

// A start and an end event per timed launch, per recorded call.
struct Profiler {
  std::mutex mu;
  unsigned mask = 0;  // bit k: time kernel k
  int ncalls = 0;
  hipEvent_t ev[kProfCalls][kProfLaunches][2] = {};
  int kid[kProfCalls][kProfLaunches];
  int nl[kProfCalls] = {};
};

Profiler &prof() {
  static Profiler p;  // created on first use, lives until the process ends
  return p;
}

}  // namespace

namespace svd {

int timing_call_begin() {
  Profiler &P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  if (!P.mask || P.ncalls >= kProfCalls) return -1;
  const int slot = P.ncalls++;
  P.nl[slot] = 0;
  return slot;
}

int timing_launch_begin(int slot, int kernel_id, hipStream_t s) {
  Profiler &P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  if (!((P.mask >> kernel_id) & 1u)) return -1;
  const int i = P.nl[slot];
  if (i >= kProfLaunches) return -1;
  hipEvent_t *e = P.ev[slot][i];
  // timing-only events: no system-scope fence (cache writeback and invalidate)
  // when recorded, which would otherwise be charged to the timed launch
  for (int j = 0; j < 2; ++j)
    if (!e[j] && hipEventCreateWithFlags(&e[j], hipEventDisableSystemFence) != hipSuccess) {
      e[j] = nullptr;
      return -1;
    }
  if (hipEventRecord(e[0], s) != hipSuccess) return -1;
  P.kid[slot][i] = -1;  // until the end event is recorded
  P.nl[slot] = i + 1;
  return i;
}

void timing_launch_end(int slot, int rec, int kernel_id, hipStream_t s) {
  Profiler &P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  if (hipEventRecord(P.ev[slot][rec][1], s) == hipSuccess) P.kid[slot][rec] = kernel_id;
}

}  // namespace svd

extern "C" {

int svd_profile_enable(unsigned kernel_mask) {
  Profiler &P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  P.mask = kernel_mask & ((1u << SVD_KERNEL_COUNT) - 1u);
  return SVD_OK;
}

int svd_profile_read(double *ms, int64_t *launches, int n) {
  if (!ms || n < 0) return SVD_EINVAL;
  Profiler &P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  for (int i = 0; i < n; ++i) {
    ms[i] = 0.0;
    if (launches) launches[i] = 0;
  }
  for (int c = 0; c < P.ncalls; ++c) {
    for (int i = 0; i < P.nl[c]; ++i) {
      const int k = P.kid[c][i];
      if (k < 0 || k >= n) continue;
      if (hipEventSynchronize(P.ev[c][i][1]) != hipSuccess) return SVD_EHIP;
      float t = 0.0f;
      if (hipEventElapsedTime(&t, P.ev[c][i][0], P.ev[c][i][1]) != hipSuccess) return SVD_EHIP;
      ms[k] += t;
      if (launches) launches[k] += 1;
    }
  }
  P.ncalls = 0;
  return SVD_OK;
}

}  // extern "C"
