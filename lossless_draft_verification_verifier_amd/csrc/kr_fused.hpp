// kr_fused.hpp -- the whole verification step in one launch.
//
// The row-statistics work streams HBM and leaves the vector ALUs half idle;
// the fp64 draw is ALU work on a small re-read.  One launch runs both, so the
// draw of early prefixes overlaps the streaming of later ones:
//
//  * Every workgroup takes a ticket from an atomic counter when it starts, and
//    the ticket names its item.  Items are row pairs (b, k, j) and draw
//    segment groups (b, kDrawGroup segments).  The order interleaves them with a lag of `lag`
//    prefixes: the row pairs of prefix b + lag come just before the draw
//    segments of prefix b, so a draw segment is handed out about when its
//    prefix's rows finish streaming.
//  * The workgroup finishing the last row pair of a prefix (an atomic count)
//    runs the selection epilogue for that prefix and then publishes a ready
//    flag (release).
//  * A draw-segment workgroup waits for its prefix's flag (acquire).  Every row
//    pair of that prefix has a smaller ticket, so its workgroup has already
//    started and runs to completion without waiting on anything: the wait
//    always ends.  It is bounded all the same: on a timeout the workgroup
//    raises a flag that stops every other wait, skips its work, and the
//    outputs of the prefixes picked afterwards become -1.
//  * The workgroup finishing the last draw segment of a prefix runs the pick,
//    recomputing exactly any segment whose list of uncertain tokens overflowed.
//
// kr_fused_init clears the counters first (a plain store loop, no memset).
#pragma once

#include "kr_draw.hpp"
#include "kr_rowstats.hpp"
#include "kr_select.hpp"

namespace svd {

constexpr int kFusedBlock = 1024;
constexpr int kFusedUnroll = 2;
constexpr int kDrawGroup = 4;  // vocabulary segments per draw item
constexpr unsigned kSpinLimit = 1u << 22;  // x ~512 cycles of sleep: about a second

template <typename E>
struct FusedArgs {
  const typename E::elem *p, *q;
  const int32_t *drafts;
  int64_t B;
  int K, gamma, V, nseg, lag;
  float tp, tq, cp, cq;
  uint64_t seed, row_base;
  int32_t *selected, *accept_len, *next_token;
  float *scores, *alpha_out;
  RowStats *stats;
  float *alpha_ws;
  DrawDesc *desc;
  DrawSeg *segs;
  DrawUnc *uncs;
  DrawMass *mass;
  unsigned *sync;  // [0] ticket, [1] timeout flag, then rows done [B], draws done [B], ready [B]
};

struct FusedItem {
  int kind;      // 0: row pair, 1: draw segment
  int64_t b;     // prefix
  int64_t idx;   // row pair index, or segment
};

// Ticket -> item.  With P row pairs and S segments per prefix and lag L:
//   phase A: the row pairs of prefixes [0, L);
//   phase B: for b in [L, B): the row pairs of prefix b, then the segments of b - L;
//   phase C: the segments of the last L prefixes.
__device__ inline FusedItem fused_decode(int64_t t, int64_t B, int64_t P, int64_t S, int64_t L) {
  const int64_t LA = L < B ? L : B;
  if (t < LA * P) return FusedItem{0, t / P, t};
  t -= LA * P;
  const int64_t nB = B - LA;
  if (t < nB * (P + S)) {
    const int64_t blk = t / (P + S), w = t - blk * (P + S);
    if (w < P) return FusedItem{0, LA + blk, (LA + blk) * P + w};
    return FusedItem{1, blk, w - P};
  }
  t -= nB * (P + S);
  return FusedItem{1, nB + t / S, t % S};
}

__global__ __launch_bounds__(256) void kr_fused_init(unsigned *__restrict__ sync, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    sync[i] = 0u;
}

// Two 1024-thread workgroups per CU (8 waves per SIMD): every path fits 64 VGPRs.
template <typename E, bool kVec>
__global__ __launch_bounds__(kFusedBlock) __attribute__((amdgpu_waves_per_eu(8))) void kr_fused(
    FusedArgs<E> a) {
  __shared__ unsigned item_s;
  __shared__ int flag_s;
  unsigned *ticket = a.sync, *timeout = a.sync + 1;
  unsigned *rows_done = a.sync + 2, *draws_done = rows_done + a.B, *ready = draws_done + a.B;
  if (threadIdx.x == 0) item_s = atomicAdd(ticket, 1u);
  __syncthreads();
  const int64_t P = (int64_t)a.K * a.gamma;
  const int S = (a.nseg + kDrawGroup - 1) / kDrawGroup;  // draw items per prefix
  const FusedItem it = fused_decode((int64_t)item_s, a.B, P, S, a.lag);

  if (it.kind == 0) {
    rowstats_item<E, kVec, kFusedBlock, kFusedUnroll>(a.p, a.q, a.drafts, a.gamma, a.V, a.cp,
                                                      a.cq, it.idx, a.stats, a.alpha_ws,
                                                      a.alpha_out);
    if (threadIdx.x == 0) {
      __threadfence();  // this row pair's statistics before the count
      flag_s = atomicAdd(&rows_done[it.b], 1u) == (unsigned)(P - 1);
    }
    __syncthreads();
    if (flag_s && threadIdx.x < 64) {
      __threadfence();  // every row pair of the prefix is visible
      select_prefix(a.alpha_ws, a.K, a.gamma, a.seed, a.row_base, it.b, a.selected, a.accept_len,
                    a.next_token, a.scores, a.desc);
      if (threadIdx.x == 0) {
        __threadfence();
        __hip_atomic_store(&ready[it.b], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return;
  }

  if (threadIdx.x == 0) {
    int ok = 0;
    for (unsigned n = 0; n < kSpinLimit; ++n) {
      if (__hip_atomic_load(&ready[it.b], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT)) {
        ok = 1;
        break;
      }
      // after one timeout nobody waits any more, so the launch drains quickly
      if (__hip_atomic_load(timeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
      __builtin_amdgcn_s_sleep(8);
    }
    if (!ok) atomicOr(timeout, 1u);
    flag_s = ok;
  }
  __syncthreads();
  const int ready_ok = flag_s;
  __syncthreads();
  if (ready_ok)
    draw_pass_item<E, kVec, true, kFusedBlock, kDrawGroup>(a.p, a.q, a.K, a.gamma, a.V, a.nseg,
                                                           a.tp, a.tq, a.stats, a.desc, a.segs,
                                                           a.uncs, it.b, (int)it.idx * kDrawGroup);
  if (threadIdx.x == 0) {
    __threadfence();  // this segment's sums before the count
    flag_s = atomicAdd(&draws_done[it.b], 1u) == (unsigned)(S - 1);
  }
  __syncthreads();
  if (!flag_s) return;
  __threadfence();  // every segment of the prefix is visible
  if (__hip_atomic_load(timeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
    if (threadIdx.x == 0) {
      if (a.selected) a.selected[it.b] = -1;
      a.accept_len[it.b] = -1;
      a.next_token[it.b] = -1;
    }
    return;
  }
  draw_pick_item<E, kVec, kFusedBlock, true>(a.p, a.q, a.K, a.gamma, a.V, a.nseg, a.tp, a.tq,
                                             a.seed, a.row_base, a.stats, a.desc, a.segs, a.uncs,
                                             a.mass, a.selected, a.accept_len, a.next_token, it.b);
}

}  // namespace svd
