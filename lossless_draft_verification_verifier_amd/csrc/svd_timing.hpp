// svd_timing.hpp -- kernel-timing hooks around the library's launches.
//
// The product library compiles every hook to nothing: it records no events
// and keeps no state between calls.  The timing build (the same sources with
// SVD_KERNEL_TIMING defined, plus svd_timing.hip) records a HIP event before
// and after each launch it is asked to time, on the launch's stream; its
// state lives in svd_timing.hip and is reached only through these hooks.
#pragma once

#include <hip/hip_runtime.h>

namespace svd {

#ifdef SVD_KERNEL_TIMING
// a record slot for one entry-point call, or -1 when timing is off or full
int timing_call_begin();
// a start event for kernel `kernel_id` of call `slot` on stream s; its record
// index, or -1 when that kernel is not timed
int timing_launch_begin(int slot, int kernel_id, hipStream_t s);
// the end event of record `rec`
void timing_launch_end(int slot, int rec, int kernel_id, hipStream_t s);
#else
inline int timing_call_begin() { return -1; }
inline int timing_launch_begin(int, int, hipStream_t) { return -1; }
inline void timing_launch_end(int, int, int, hipStream_t) {}
#endif

// One entry-point call's handle on the hooks (a no-op in the product build).
struct CallTimer {
  int slot = timing_call_begin();
  int begin(int kernel_id, hipStream_t s) {
    return slot < 0 ? -1 : timing_launch_begin(slot, kernel_id, s);
  }
  void end(int rec, int kernel_id, hipStream_t s) {
    if (rec >= 0) timing_launch_end(slot, rec, kernel_id, s);
  }
};

}  // namespace svd
