// svd_api.hip -- the C ABI declared in include/svd.h: argument checks,
// workspace layout and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <tuple>
#include <utility>

#include "svd.h"
#include "svd_timing.h"
#include "svd_timing.hpp"
#include "kr_adl.hpp"
#include "kr_beam.hpp"
#include "kr_beta.hpp"
#include "kr_cps.hpp"
#include "kr_draw.hpp"
#include "kr_rows.hpp"
#include "kr_rowstats.hpp"
#include "kr_select.hpp"

namespace {

using namespace svd;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Layout {
  size_t stats, alpha, desc, segs, uncs, mass, mlen, alive, live, counts, part, pstat, flags,
      total;
  int seg, nseg;
};

// Tokens per draw segment: the pass runs one workgroup per (prefix, segment)
// and about 1536 of them are resident at once, so a batch that would fill
// fewer than half of those with segments of kDrawSeg tokens takes segments of
// kDrawSegSmall (a shorter serial run per workgroup, more workgroups).
constexpr int64_t kDrawSmallBelow = 768;
int draw_seg(int64_t B, int32_t V) {
  const int64_t nbig = ((int64_t)V + kDrawSeg - 1) / kDrawSeg;
  return B * nbig < kDrawSmallBelow ? kDrawSegSmall : kDrawSeg;
}

// Split rows: at most this many (row pair, slice) records per launch.
constexpr int kPartCap = 4096;
static_assert(kLiveGrid <= kPartCap, "a live-list launch writes up to kLiveGrid records");
constexpr int kLiveCounts = SVD_MAX_GAMMA + 1;  // chunk counters of an early exit
constexpr int64_t kLiveWholeRows = 512;  // a first chunk of this many row pairs streams whole rows
constexpr int64_t kSplitRows = 1024;    // launches with fewer row pairs are split
constexpr int64_t kSplitTarget = 2048;  // slice workgroups to aim for

bool sizes_ok(int64_t B, int32_t K, int32_t G, int32_t V) {
  if (B < 1 || K < 1 || G < 1 || V < 1) return false;
  if (K > SVD_MAX_K || G > SVD_MAX_GAMMA) return false;
  const int seg = draw_seg(B, V);
  const int64_t nseg = ((int64_t)V + seg - 1) / seg;
  const int64_t lim = (int64_t)1 << 31;
  if (B >= lim / ((int64_t)K * G)) return false;  // B*K*gamma workgroups
  if (B >= lim / nseg) return false;              // B*nseg workgroups
  return true;
}

// np, nq: pool rows of the shared-row entry point (0 for the dense layout)
Layout layout(int64_t B, int32_t K, int32_t G, int32_t V, int64_t np = 0, int64_t nq = 0) {
  Layout L{};
  const size_t rp = (size_t)B * K * G;
  L.seg = draw_seg(B, V);
  L.nseg = (int)(((int64_t)V + L.seg - 1) / L.seg);
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
  L.mlen = off;
  off = align_up(off + (size_t)B * K * sizeof(int32_t));
  L.alive = off;
  off = align_up(off + (size_t)B * sizeof(uint32_t));
  L.live = off;  // early exit: two lists of live prefixes, and a counter per chunk
  off = align_up(off + (size_t)2 * B * sizeof(int32_t));
  L.counts = off;
  off = align_up(off + (size_t)kLiveCounts * sizeof(uint32_t));
  L.part = off;
  off = align_up(off + (size_t)kPartCap * sizeof(PartStats));
  L.pstat = off;
  off = align_up(off + (size_t)(np + nq) * sizeof(PoolStat));
  L.flags = off;
  off = align_up(off + (size_t)(np + nq) * sizeof(uint32_t));
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

// Index tables of the shared-row layout ([B][K][gamma+1] and [B][K][gamma]);
// null tables mean the dense layout.
struct RowIndex {
  const int32_t *p;
  const int32_t *q;
};

// Everything the launch chain reads and writes.
template <typename E>
struct Batch {
  const typename E::elem *p, *q;
  const int32_t *drafts;
  int64_t B;
  int K, G, V, seg, nseg;
  float tp, tq, cp, cq;
  uint64_t seed, row_base;
  bool greedy;  // greedy acceptance: alpha = p(x), q unused
  RowIndex ix;  // shared rows: p and q are pools of np and nq rows (ix.p null: dense)
  int64_t np, nq;
  PoolStat *pstat;
  uint32_t *flags;
  bool windowed, early;  // ragged / EOS-aware windows; K == 1 streamed up to the first rejection
  const int32_t *gamma_b;
  int eos;
  int32_t *mlen;
  uint32_t *alive;
  int32_t *live;     // early exit: two lists of B prefixes
  uint32_t *counts;  // early exit: live prefixes per chunk
  PartStats *part;
  bool vec;  // 16-byte loads
  bool fuse_select;  // the selection runs in the launch that forms alpha (kr_combine_select, kr_alpha_select)
  int32_t *selected, *accept_len, *next_token;
  float *scores, *alpha, *beta;
  RowStats *stats;
  float *alpha_ws;
  DrawDesc *desc;
  DrawSeg *segs;
  DrawUnc *uncs;
  DrawMass *mass;
};

#define SVD_LAUNCH(tm, kid, stream, ...)                            \
  do {                                                              \
    const int rec_ = (tm).begin((kid), (stream));                   \
    if (launch(__VA_ARGS__) != hipSuccess) return SVD_EHIP;         \
    (tm).end(rec_, (kid), (stream));                                \
  } while (0)

// Lattice launches of fewer rows are split (a whole row per workgroup keeps
// up four loads in flight per thread and does its selection once).
constexpr int64_t kLatticeSplitRows = 128;

// Positions per chunk when one draft per prefix is streamed up to its first
// rejection: enough workgroups per launch to fill the GPU about once.
int early_chunk(int64_t B, int G) {
  const int64_t want = (512 + B - 1) / B;
  return (int)std::max<int64_t>(1, std::min<int64_t>(want, G));
}

// Length of chunk c: J positions for the first two chunks, then twice the
// chunk before, at most cap.  Fewer prefixes reach each later chunk, so
// reading a few positions past a rejection there costs less than another
// round of launches.
int early_chunk_len(int c, int J, int cap) {
  return c < 2 ? J : std::max(J, std::min(J << std::min(c - 1, 20), cap));
}

// chunks of a window of G positions
int early_chunks(int G, int J, int cap) {
  int n = 0;
  for (int j0 = 0; j0 < G; j0 += early_chunk_len(n, J, cap)) ++n;
  return n;
}

// Split rows: slices per row pair (1: not split) and the slice length for a
// launch of `rows` row pairs.
template <typename E>
void split_plan(const Batch<E> &a, int64_t rows, int &S, int &slice) {
  S = 1;
  slice = a.V;
  if (rows >= kSplitRows) return;
  const int unit = a.vec ? E::kPerVec : 1;  // elements per load
  const int64_t units = a.V / unit;
  const int64_t most = std::max<int64_t>(1, units / (2 * kSplitBlock));
  const int64_t want = std::min<int64_t>((kSplitTarget + rows - 1) / rows, kPartCap / rows);
  const int64_t s_try = std::max<int64_t>(1, std::min(most, want));
  slice = (int)((units + s_try - 1) / s_try) * unit;
  S = (a.V + slice - 1) / slice;
}

// the selection's arguments for a batch
template <typename E>
SelectArgs make_select(const Batch<E> &a) {
  return SelectArgs{(const float *)a.alpha_ws, (const RowStats *)a.stats, a.drafts,
                    (int)a.greedy, a.ix.p, a.greedy ? nullptr : a.ix.q, a.np,
                    Window{a.windowed ? (const int32_t *)a.mlen : nullptr, a.gamma_b, a.eos,
                           (int)a.early},
                    a.K, a.G, a.seed, a.row_base, a.selected, a.accept_len, a.next_token,
                    a.scores};
}

// one workgroup per row pair (positions [j0, j0 + jn) of every draft); short
// rows take smaller workgroups
template <typename E, bool kVec, bool kGreedy, int NT>
int launch_rowstats_nt(const Batch<E> &a, hipStream_t s, CallTimer &tm, unsigned grid,
                       const int32_t *mlen, const uint32_t *alive, int j0, int jn) {
  SVD_LAUNCH(tm, SVD_KERNEL_ROWSTATS, s, kr_rowstats<E, kVec, kGreedy, NT>, dim3(grid), dim3(NT),
             s, a.p, a.q, a.drafts, a.G, a.V, a.cp, a.cq, a.stats, a.alpha_ws, a.alpha, mlen,
             alive, j0, jn);
  return SVD_OK;
}
template <typename E, bool kVec>
int launch_rowstats(const Batch<E> &a, hipStream_t s, CallTimer &tm, unsigned grid,
                    const int32_t *mlen, const uint32_t *alive, int j0, int jn) {
  const bool short_rows = (int64_t)a.V * (int64_t)sizeof(typename E::elem) < kShortRowBytes;
  if (a.greedy)
    return short_rows
               ? launch_rowstats_nt<E, kVec, true, kShortRowBlock>(a, s, tm, grid, mlen, alive,
                                                                   j0, jn)
               : launch_rowstats_nt<E, kVec, true, kRowBlock>(a, s, tm, grid, mlen, alive, j0, jn);
  return short_rows
             ? launch_rowstats_nt<E, kVec, false, kShortRowBlock>(a, s, tm, grid, mlen, alive, j0,
                                                                  jn)
             : launch_rowstats_nt<E, kVec, false, kRowBlock>(a, s, tm, grid, mlen, alive, j0, jn);
}

// row statistics and alpha (and the optional overlap mass) of a batch
template <typename E, bool kVec>
int enqueue_rows(const Batch<E> &a, hipStream_t s, CallTimer &tm) {
  const unsigned rp = (unsigned)(a.B * a.K * a.G);
  if (a.ix.p) {  // shared rows: statistics once per pool row read, then alpha per position
    const int64_t nrows = a.np + (a.greedy ? 0 : a.nq);
    const unsigned gp = (unsigned)((rp + kBlock - 1) / kBlock);
    const unsigned gf = (unsigned)std::min<int64_t>((nrows + kBlock - 1) / kBlock, 4096);
    if (nrows <= kMarkLdsRows) {
      SVD_LAUNCH(tm, SVD_KERNEL_MARK, s, kr_mark_rows_one, dim3(1), dim3(1024), s, a.ix.p,
                 a.greedy ? nullptr : a.ix.q, (int64_t)rp, a.G, a.np, a.nq, nrows, a.flags);
    } else {
      SVD_LAUNCH(tm, SVD_KERNEL_MARK, s, kr_fill_u32, dim3(gf), dim3(kBlock), s, a.flags, nrows,
                 0u);
      SVD_LAUNCH(tm, SVD_KERNEL_MARK, s, kr_mark_rows, dim3(gp), dim3(kBlock), s, a.ix.p,
                 a.greedy ? nullptr : a.ix.q, (int64_t)rp, a.G, a.np, a.nq, a.flags);
    }
    if ((int64_t)a.V * (int64_t)sizeof(typename E::elem) < kShortRowBytes)
      SVD_LAUNCH(tm, SVD_KERNEL_POOL_STATS, s, kr_pool_stats<E, kVec, kShortRowBlock>,
                 dim3((unsigned)nrows), dim3(kShortRowBlock), s, a.p, a.q, a.np, a.V, a.cp, a.cq,
                 (const uint32_t *)a.flags, a.pstat);
    else
      SVD_LAUNCH(tm, SVD_KERNEL_POOL_STATS, s, kr_pool_stats<E, kVec>, dim3((unsigned)nrows),
                 dim3(kRowBlock), s, a.p, a.q, a.np, a.V, a.cp, a.cq, (const uint32_t *)a.flags,
                 a.pstat);
    if (a.fuse_select) {  // alpha and the selection, a workgroup per prefix
      const SelectArgs sel = make_select(a);
      const int kg = a.K * a.G;
      const dim3 tb((unsigned)std::min(kAlphaSelectMax, std::max(64, (kg + 63) / 64 * 64)));
      if (a.greedy)
        SVD_LAUNCH(tm, SVD_KERNEL_ALPHA_ROWS, s, kr_alpha_select<E, true>, dim3((unsigned)a.B),
                   tb, s, a.p, a.q, a.V, a.nq, a.cp, a.cq, (const PoolStat *)a.pstat, a.stats,
                   a.alpha_ws, a.alpha, sel, a.desc);
      else
        SVD_LAUNCH(tm, SVD_KERNEL_ALPHA_ROWS, s, kr_alpha_select<E, false>, dim3((unsigned)a.B),
                   tb, s, a.p, a.q, a.V, a.nq, a.cp, a.cq, (const PoolStat *)a.pstat, a.stats,
                   a.alpha_ws, a.alpha, sel, a.desc);
      return SVD_OK;
    }
    if (a.greedy)
      SVD_LAUNCH(tm, SVD_KERNEL_ALPHA_ROWS, s, kr_alpha_rows<E, true>, dim3(gp), dim3(kBlock), s,
                 a.p, a.q, a.ix.p, a.ix.q, a.drafts, (int64_t)rp, a.G, a.V, a.np, a.nq, a.cp,
                 a.cq, (const PoolStat *)a.pstat, a.stats, a.alpha_ws, a.alpha);
    else
      SVD_LAUNCH(tm, SVD_KERNEL_ALPHA_ROWS, s, kr_alpha_rows<E, false>, dim3(gp), dim3(kBlock), s,
                 a.p, a.q, a.ix.p, a.ix.q, a.drafts, (int64_t)rp, a.G, a.V, a.np, a.nq, a.cp,
                 a.cq, (const PoolStat *)a.pstat, a.stats, a.alpha_ws, a.alpha);
    return SVD_OK;
  }
  // early exit over a live list: the batch's chunks are split rows (few row
  // pairs per chunk) and the rows can be cut in more than one slice
  const int J = a.early ? early_chunk(a.B, a.G) : a.G;
  const int unit = a.vec ? E::kPerVec : 1;  // elements per load
  const int units = a.V / unit;
  const int smax = (int)std::max<int64_t>(1, units / (2 * kSplitBlock));
  const bool live = a.early && a.B * J < kSplitRows && smax > 1;
  // a live-list chunk of the whole batch must fit the fixed grid (one slice
  // per row at most)
  const int cap = live ? (int)std::max<int64_t>(J, kLiveGrid / a.B) : a.G;
  const int nchunks = a.early ? early_chunks(a.G, J, cap) : 1;
  const int32_t *mlen = nullptr;
  if (a.windowed) {
    const int64_t bk = a.B * a.K;
    const int64_t nt = live ? std::max<int64_t>(bk, nchunks + 1) : bk;
    SVD_LAUNCH(tm, SVD_KERNEL_SELECT, s, kr_window, dim3((unsigned)((nt + kBlock - 1) / kBlock)),
               dim3(kBlock), s, a.drafts, a.gamma_b, a.eos, bk, a.K, a.G, a.mlen,
               live ? a.live : nullptr, live ? a.counts : nullptr, live ? nchunks + 1 : 0);
    mlen = a.mlen;
  }
  if (live) {
    // chunk c reads list c % 2 and its counter c, and writes the next ones
    const unsigned gw = (unsigned)((a.B * 64 + kBlock - 1) / kBlock);  // a wave per prefix
    for (int c = 0, j0 = 0; c < nchunks; j0 += early_chunk_len(c, J, cap), ++c) {
      const int Jc = std::min(early_chunk_len(c, J, cap), a.G - j0);
      const int32_t *cur = a.live + (c % 2) * a.B;
      int32_t *next = a.live + ((c + 1) % 2) * a.B;
      const uint32_t *cnt = a.counts + c;
      uint32_t *cnt_next = c + 1 < nchunks ? a.counts + c + 1 : nullptr;
      // the first chunk holds every prefix: with enough row pairs to give each
      // CU two, it streams whole rows (kr_rowstats), and the merge only tests
      const bool whole = c == 0 && a.B * Jc >= kLiveWholeRows;
      const PartStats *part = whole ? nullptr : a.part;
      if (whole) {
        {
          const int rc = launch_rowstats<E, kVec>(a, s, tm, (unsigned)(a.B * Jc), mlen, nullptr, 0,
                                                  Jc);
          if (rc != SVD_OK) return rc;
        }
        if (a.greedy)
          SVD_LAUNCH(tm, SVD_KERNEL_COMBINE, s, kr_combine_advance<E, true>, dim3(gw),
                     dim3(kBlock), s, a.p, a.q, a.drafts, a.G, a.V, a.cp, a.cq, units, unit, smax,
                     mlen, cur, cnt, j0, Jc, part, a.stats, a.alpha_ws, a.alpha, a.seed,
                     a.row_base, next, cnt_next);
        else
          SVD_LAUNCH(tm, SVD_KERNEL_COMBINE, s, kr_combine_advance<E, false>, dim3(gw),
                     dim3(kBlock), s, a.p, a.q, a.drafts, a.G, a.V, a.cp, a.cq, units, unit, smax,
                     mlen, cur, cnt, j0, Jc, part, a.stats, a.alpha_ws, a.alpha, a.seed,
                     a.row_base, next, cnt_next);
        continue;
      }
      if (a.greedy) {
        SVD_LAUNCH(tm, SVD_KERNEL_ROWSTATS_LIVE, s, kr_rowstats_live<E, kVec, true>,
                   dim3(kLiveGrid), dim3(kSplitBlock), s, a.p, a.q, a.G, a.V, a.cp, a.cq, units,
                   unit, smax, mlen, cur, cnt, j0, Jc, a.part);
        SVD_LAUNCH(tm, SVD_KERNEL_COMBINE, s, kr_combine_advance<E, true>, dim3(gw),
                   dim3(kBlock), s, a.p, a.q, a.drafts, a.G, a.V, a.cp, a.cq, units, unit, smax,
                   mlen, cur, cnt, j0, Jc, (const PartStats *)a.part, a.stats, a.alpha_ws,
                   a.alpha, a.seed, a.row_base, next, cnt_next);
      } else {
        SVD_LAUNCH(tm, SVD_KERNEL_ROWSTATS_LIVE, s, kr_rowstats_live<E, kVec, false>,
                   dim3(kLiveGrid), dim3(kSplitBlock), s, a.p, a.q, a.G, a.V, a.cp, a.cq, units,
                   unit, smax, mlen, cur, cnt, j0, Jc, a.part);
        SVD_LAUNCH(tm, SVD_KERNEL_COMBINE, s, kr_combine_advance<E, false>, dim3(gw),
                   dim3(kBlock), s, a.p, a.q, a.drafts, a.G, a.V, a.cp, a.cq, units, unit, smax,
                   mlen, cur, cnt, j0, Jc, (const PartStats *)a.part, a.stats, a.alpha_ws,
                   a.alpha, a.seed, a.row_base, next, cnt_next);
      }
    }
    return SVD_OK;
  }
  // the positions [j0, j0 + jn) of every draft
  auto stream_rows = [&](int j0, int jn, const uint32_t *alive) -> int {
    const int64_t rows = a.B * a.K * jn;
    int S, slice;
    split_plan<E>(a, rows, S, slice);
    if (S > 1) {
      const dim3 grid((unsigned)(rows * S));
      if (a.greedy)
        SVD_LAUNCH(tm, SVD_KERNEL_ROWSTATS_SPLIT, s, kr_rowstats_split<E, kVec, true>, grid,
                   dim3(kSplitBlock), s, a.p, a.q, a.G, a.V, a.cp, a.cq, S, slice, mlen, alive, j0,
                   jn, a.part);
      else
        SVD_LAUNCH(tm, SVD_KERNEL_ROWSTATS_SPLIT, s, kr_rowstats_split<E, kVec, false>, grid,
                   dim3(kSplitBlock), s, a.p, a.q, a.G, a.V, a.cp, a.cq, S, slice, mlen, alive, j0,
                   jn, a.part);
      if (a.fuse_select) {  // the whole window at once, few rows per prefix
        const SelectArgs sel = make_select(a);
        const dim3 gb((unsigned)a.B), tb((unsigned)(64 * a.K * a.G));
        if (a.greedy)
          SVD_LAUNCH(tm, SVD_KERNEL_COMBINE, s, kr_combine_select<E, true>, gb, tb, s, a.p, a.q,
                     a.V, a.cp, a.cq, S, (const PartStats *)a.part, a.stats, a.alpha_ws, a.alpha,
                     sel, a.desc);
        else
          SVD_LAUNCH(tm, SVD_KERNEL_COMBINE, s, kr_combine_select<E, false>, gb, tb, s, a.p,
                     a.q, a.V, a.cp, a.cq, S, (const PartStats *)a.part, a.stats, a.alpha_ws,
                     a.alpha, sel, a.desc);
        return SVD_OK;
      }
      const dim3 gc((unsigned)((rows * 64 + kBlock - 1) / kBlock));  // a wave per row
      if (a.greedy)
        SVD_LAUNCH(tm, SVD_KERNEL_COMBINE, s, kr_rowstats_combine<E, true>, gc, dim3(kBlock), s,
                   a.p, a.q, a.drafts, rows, a.G, a.V, a.cp, a.cq, S, mlen, alive, j0, jn,
                   (const PartStats *)a.part, a.stats, a.alpha_ws, a.alpha);
      else
        SVD_LAUNCH(tm, SVD_KERNEL_COMBINE, s, kr_rowstats_combine<E, false>, gc, dim3(kBlock), s,
                   a.p, a.q, a.drafts, rows, a.G, a.V, a.cp, a.cq, S, mlen, alive, j0, jn,
                   (const PartStats *)a.part, a.stats, a.alpha_ws, a.alpha);
      return SVD_OK;
    }
    return launch_rowstats<E, kVec>(a, s, tm, (unsigned)rows, mlen, alive, j0, jn);
  };
  if (!a.early) {
    const int rc = stream_rows(0, a.G, nullptr);
    if (rc != SVD_OK) return rc;
  } else {
    // one draft per prefix, positions in chunks of J; a draft leaves the
    // stream after the chunk holding its first rejection
    const unsigned gb = (unsigned)((a.B + kBlock - 1) / kBlock);
    SVD_LAUNCH(tm, SVD_KERNEL_SELECT, s, kr_fill_u32, dim3(gb), dim3(kBlock), s, a.alive, a.B, 1u);
    for (int c = 0, j0 = 0; j0 < a.G; j0 += early_chunk_len(c, J, cap), ++c) {
      const int Jc = std::min(early_chunk_len(c, J, cap), a.G - j0);
      const int rc = stream_rows(j0, Jc, a.alive);
      if (rc != SVD_OK) return rc;
      if (j0 + Jc < a.G)
        SVD_LAUNCH(tm, SVD_KERNEL_SELECT, s, kr_advance, dim3(gb), dim3(kBlock), s,
                   (const float *)a.alpha_ws, (const int32_t *)a.mlen, a.B, a.G, j0, Jc, a.seed,
                   a.row_base, a.alive);
    }
  }
  if (a.beta) {
    // few row pairs: slices, as for the statistics, then their sums added
    int S, slice;
    split_plan<E>(a, rp, S, slice);
    float *part = reinterpret_cast<float *>(a.part);  // free again once the stream is merged
    SVD_LAUNCH(tm, SVD_KERNEL_BETA, s, kr_beta<E, kVec>, dim3((unsigned)(rp * S)), dim3(kBlock),
               s, a.p, a.q, a.G, a.V, a.cp, a.cq, (const RowStats *)a.stats, S, slice, a.beta,
               part);
    if (S > 1)
      SVD_LAUNCH(tm, SVD_KERNEL_BETA_COMBINE, s, kr_beta_combine,
                 dim3((unsigned)((rp + kBlock - 1) / kBlock)), dim3(kBlock), s, (int64_t)rp, S,
                 (const float *)part, a.beta);
  }
  return SVD_OK;
}

// the draw's pass and pick, in segments of SEG tokens
template <typename E, bool kVec, int SEG>
int enqueue_pass_pick(const Batch<E> &a, hipStream_t s, CallTimer &tm) {
  const unsigned nb = (unsigned)a.B;
  const unsigned nbs = (unsigned)(a.B * a.nseg);
  SVD_LAUNCH(tm, SVD_KERNEL_DRAW_PASS, s, kr_draw_pass<E, kVec, SEG>, dim3(nbs),
             dim3(kPassBlock), s, a.p, a.q, a.V, a.nseg, a.tp, a.tq, (const DrawDesc *)a.desc,
             a.segs, a.uncs);
  SVD_LAUNCH(tm, SVD_KERNEL_DRAW_PICK, s, kr_draw_pick<E, kVec, SEG>, dim3(nb),
             dim3(kPickBlock), s, a.p, a.q, a.V, a.nseg, a.tp, a.tq, a.seed, a.row_base,
             (const DrawDesc *)a.desc, (const DrawSeg *)a.segs, (const DrawUnc *)a.uncs, a.mass,
             a.selected, a.accept_len, a.next_token);
  return SVD_OK;
}

// selection, first rejection and the draw of a batch whose statistics are done
template <typename E, bool kVec>
int enqueue_draw(const Batch<E> &a, hipStream_t s, CallTimer &tm) {
  const unsigned nb = (unsigned)a.B;
  if (!a.fuse_select)
    SVD_LAUNCH(tm, SVD_KERNEL_SELECT, s, kr_select, dim3(nb), dim3(64), s, make_select(a), a.desc);
  if (a.seg == kDrawSeg)
    return enqueue_pass_pick<E, kVec, kDrawSeg>(a, s, tm);
  return enqueue_pass_pick<E, kVec, kDrawSegSmall>(a, s, tm);
}

// The arguments of one entry-point call.
struct Call {
  const void *p, *q;  // logits (dense), or row pools when p_index is set
  const int32_t *drafts;
  svd_dtype_t dtype;
  int64_t B;
  int32_t K, G, V;
  float tp, tq;
  uint64_t seed, row_base;
  bool greedy;
  const int32_t *p_index, *q_index;  // shared rows (null: dense layout)
  int64_t np, nq;
  bool windowed, early;  // ragged / EOS-aware windows; stream up to the first rejection
  const int32_t *gamma_b;
  int32_t eos;
  int32_t *selected, *accept_len, *next_token;
  float *scores, *alpha, *beta;
  void *workspace;
  size_t workspace_bytes;
  void *stream;
};

template <typename E, bool kVec>
int run(const Call &c) {
  using T = typename E::elem;
  const Layout Lo = layout(c.B, c.K, c.G, c.V, c.np, c.nq);
  char *ws = static_cast<char *>(c.workspace);
  Batch<E> a;
  a.p = static_cast<const T *>(c.p);
  a.q = static_cast<const T *>(c.q);
  a.drafts = c.drafts;
  a.B = c.B;
  a.K = c.K;
  a.G = c.G;
  a.V = c.V;
  a.seg = Lo.seg;
  a.nseg = Lo.nseg;
  a.tp = c.tp;
  a.tq = c.tq;
  // log2(e) / T folded into one factor per row: exp(z/T) = exp2(z * c)
  a.cp = (float)(1.4426950408889634 / (double)c.tp);
  a.cq = (float)(1.4426950408889634 / (double)c.tq);
  a.seed = c.seed;
  a.row_base = c.row_base;
  a.greedy = c.greedy;
  a.ix = RowIndex{c.p_index, c.q_index};
  a.np = c.np;
  a.nq = c.nq;
  a.windowed = c.windowed;
  a.early = c.early;
  a.gamma_b = c.gamma_b;
  a.eos = c.windowed ? c.eos : -1;
  a.mlen = reinterpret_cast<int32_t *>(ws + Lo.mlen);
  a.part = reinterpret_cast<PartStats *>(ws + Lo.part);
  a.vec = kVec;
  a.alive = reinterpret_cast<uint32_t *>(ws + Lo.alive);
  a.live = reinterpret_cast<int32_t *>(ws + Lo.live);
  a.counts = reinterpret_cast<uint32_t *>(ws + Lo.counts);
  a.pstat = reinterpret_cast<PoolStat *>(ws + Lo.pstat);
  a.flags = reinterpret_cast<uint32_t *>(ws + Lo.flags);
  a.selected = c.selected;
  a.accept_len = c.accept_len;
  a.next_token = c.next_token;
  a.scores = c.scores;
  a.alpha = c.alpha;
  a.beta = c.beta;
  a.stats = reinterpret_cast<RowStats *>(ws + Lo.stats);
  a.alpha_ws = reinterpret_cast<float *>(ws + Lo.alpha);
  a.desc = reinterpret_cast<DrawDesc *>(ws + Lo.desc);
  a.segs = reinterpret_cast<DrawSeg *>(ws + Lo.segs);
  a.uncs = reinterpret_cast<DrawUnc *>(ws + Lo.uncs);
  a.mass = reinterpret_cast<DrawMass *>(ws + Lo.mass);
  // few rows per prefix, dense, the whole window in one split launch: the
  // selection joins the merge of the split rows
  int S_all, slice_all;
  split_plan<E>(a, a.B * a.K * a.G, S_all, slice_all);
  // the selection runs in the launch that forms alpha: split rows merged a
  // prefix per workgroup, or shared rows with few positions per prefix
  a.fuse_select = (!a.ix.p && !a.early && S_all > 1 && a.K * a.G <= kFuseRows) ||
                  (a.ix.p && a.K * a.G <= kAlphaSelectMax);

  hipStream_t stream = static_cast<hipStream_t>(c.stream);
  CallTimer tm;
  const int rc = enqueue_rows<E, kVec>(a, stream, tm);
  return rc != SVD_OK ? rc : enqueue_draw<E, kVec>(a, stream, tm);
}

// A temperature must be finite and positive, and log2(e) / T (the fp32 factor
// of every exp2 argument) finite: T below about 4.2e-39 is rejected.
bool temp_ok(float t) {
  if (!(std::isfinite(t) && t > 0.0f)) return false;
  const float c = (float)(1.4426950408889634 / (double)t);
  return std::isfinite(c);
}

bool pools_ok(int64_t np, int64_t nq, bool greedy) {
  const int64_t lim = (int64_t)1 << 30;
  return np >= 1 && np < lim && nq >= (greedy ? 0 : 1) && nq < lim;
}

int dispatch(const Call &c) {
  const bool rows = c.p_index != nullptr;
  if (!c.p || (!c.q && !c.greedy) || !c.drafts || !c.accept_len || !c.next_token ||
      !c.workspace || (rows && !c.greedy && !c.q_index))
    return SVD_EINVAL;
  if (c.dtype != SVD_F32 && c.dtype != SVD_BF16) return SVD_EDTYPE;
  if (!sizes_ok(c.B, c.K, c.G, c.V) || !temp_ok(c.tp) || !temp_ok(c.tq)) return SVD_EINVAL;
  if (rows && !pools_ok(c.np, c.nq, c.greedy)) return SVD_EINVAL;
  if (c.windowed && (rows || c.beta || c.eos >= c.V)) return SVD_EINVAL;
  if (c.early && (!c.windowed || c.K != 1 || c.scores)) return SVD_EINVAL;
  if (((uintptr_t)c.workspace) % kAlign != 0) return SVD_EINVAL;
  if (c.workspace_bytes < layout(c.B, c.K, c.G, c.V, c.np, c.nq).total) return SVD_EWORKSPACE;
  const size_t es = c.dtype == SVD_F32 ? 4 : 2;
  // 16-byte loads need every row to start 16-byte aligned
  const bool vec = ((size_t)c.V * es) % 16 == 0 && ((uintptr_t)c.p) % 16 == 0 &&
                   ((uintptr_t)c.q) % 16 == 0;
  if (c.dtype == SVD_BF16) return vec ? run<BF16, true>(c) : run<BF16, false>(c);
  return vec ? run<F32, true>(c) : run<F32, false>(c);
}

Call make_call(const void *p, const void *q, const int32_t *drafts, svd_dtype_t dtype, int64_t B,
               int32_t K, int32_t G, int32_t V, float tp, float tq, uint64_t seed,
               uint64_t row_base, bool greedy, int32_t *selected, int32_t *accept_len,
               int32_t *next_token, float *scores, float *alpha, float *beta, void *workspace,
               size_t workspace_bytes, void *stream) {
  Call c{};
  c.p = p;
  c.q = q;
  c.drafts = drafts;
  c.dtype = dtype;
  c.B = B;
  c.K = K;
  c.G = G;
  c.V = V;
  c.tp = tp;
  c.tq = tq;
  c.seed = seed;
  c.row_base = row_base;
  c.greedy = greedy;
  c.selected = selected;
  c.accept_len = accept_len;
  c.next_token = next_token;
  c.scores = scores;
  c.alpha = alpha;
  c.beta = beta;
  c.workspace = workspace;
  c.workspace_bytes = workspace_bytes;
  c.stream = stream;
  c.eos = -1;
  return c;
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
  return dispatch(make_call(p_logits, q_logits, draft, dtype, B, 1, gamma, V, temp_p, temp_q,
                            seed, row_base, false, nullptr, accept_len, next_token, nullptr,
                            alpha, beta, workspace, workspace_bytes, hip_stream));
}

int svd_select_and_verify(const void *p_logits, const void *q_logits, const int32_t *drafts,
                          svd_dtype_t dtype, int64_t B, int32_t K, int32_t gamma, int32_t V,
                          float temp_p, float temp_q, uint64_t seed, uint64_t row_base,
                          int32_t *selected, int32_t *accept_len, int32_t *next_token,
                          float *scores, float *alpha, float *beta, void *workspace,
                          size_t workspace_bytes, void *hip_stream) {
  if (!selected) return SVD_EINVAL;
  return dispatch(make_call(p_logits, q_logits, drafts, dtype, B, K, gamma, V, temp_p, temp_q,
                            seed, row_base, false, selected, accept_len, next_token, scores,
                            alpha, beta, workspace, workspace_bytes, hip_stream));
}

int svd_greedy_verify(const void *p_logits, const int32_t *draft, svd_dtype_t dtype, int64_t B,
                      int32_t gamma, int32_t V, float temp_p, uint64_t seed, uint64_t row_base,
                      int32_t *accept_len, int32_t *next_token, float *alpha, void *workspace,
                      size_t workspace_bytes, void *hip_stream) {
  return dispatch(make_call(p_logits, nullptr, draft, dtype, B, 1, gamma, V, temp_p, temp_p,
                            seed, row_base, true, nullptr, accept_len, next_token, nullptr, alpha,
                            nullptr, workspace, workspace_bytes, hip_stream));
}

int svd_greedy_select_and_verify(const void *p_logits, const int32_t *drafts, svd_dtype_t dtype,
                                 int64_t B, int32_t K, int32_t gamma, int32_t V, float temp_p,
                                 uint64_t seed, uint64_t row_base, int32_t *selected,
                                 int32_t *accept_len, int32_t *next_token, float *scores,
                                 float *alpha, void *workspace, size_t workspace_bytes,
                                 void *hip_stream) {
  if (!selected) return SVD_EINVAL;
  return dispatch(make_call(p_logits, nullptr, drafts, dtype, B, K, gamma, V, temp_p, temp_p,
                            seed, row_base, true, selected, accept_len, next_token, scores, alpha,
                            nullptr, workspace, workspace_bytes, hip_stream));
}

size_t svd_rows_workspace_bytes(int64_t B, int32_t K, int32_t gamma, int32_t V,
                                int64_t n_p_rows, int64_t n_q_rows) {
  if (!sizes_ok(B, K, gamma, V) || !pools_ok(n_p_rows, n_q_rows, true)) return 0;
  return layout(B, K, gamma, V, n_p_rows, n_q_rows).total;
}

int svd_select_and_verify_rows(svd_rule_t rule, const void *p_rows, int64_t n_p_rows,
                               const int32_t *p_index, const void *q_rows, int64_t n_q_rows,
                               const int32_t *q_index, const int32_t *drafts, svd_dtype_t dtype,
                               int64_t B, int32_t K, int32_t gamma, int32_t V, float temp_p,
                               float temp_q, uint64_t seed, uint64_t row_base, int32_t *selected,
                               int32_t *accept_len, int32_t *next_token, float *scores,
                               float *alpha, void *workspace, size_t workspace_bytes,
                               void *hip_stream) {
  if (rule != SVD_RULE_STANDARD && rule != SVD_RULE_GREEDY) return SVD_EINVAL;
  if (!selected || !p_index) return SVD_EINVAL;
  const bool greedy = rule == SVD_RULE_GREEDY;
  Call c = make_call(p_rows, greedy ? nullptr : q_rows, drafts, dtype, B, K, gamma, V, temp_p,
                     greedy ? temp_p : temp_q, seed, row_base, greedy, selected, accept_len,
                     next_token, scores, alpha, nullptr, workspace, workspace_bytes, hip_stream);
  c.p_index = p_index;
  c.q_index = greedy ? nullptr : q_index;
  c.np = n_p_rows;
  c.nq = greedy ? 0 : n_q_rows;
  return dispatch(c);
}

int svd_verify_window(svd_rule_t rule, const void *p_logits, const void *q_logits,
                      const int32_t *drafts, const int32_t *gamma_b, int32_t eos,
                      int32_t early_exit, svd_dtype_t dtype, int64_t B, int32_t K, int32_t gamma,
                      int32_t V, float temp_p, float temp_q, uint64_t seed, uint64_t row_base,
                      int32_t *selected, int32_t *accept_len, int32_t *next_token, float *scores,
                      float *alpha, void *workspace, size_t workspace_bytes, void *hip_stream) {
  if (rule != SVD_RULE_STANDARD && rule != SVD_RULE_GREEDY) return SVD_EINVAL;
  if (!selected) return SVD_EINVAL;
  const bool greedy = rule == SVD_RULE_GREEDY;
  Call c = make_call(p_logits, greedy ? nullptr : q_logits, drafts, dtype, B, K, gamma, V, temp_p,
                     greedy ? temp_p : temp_q, seed, row_base, greedy, selected, accept_len,
                     next_token, scores, alpha, nullptr, workspace, workspace_bytes, hip_stream);
  c.windowed = true;
  c.early = early_exit != 0;
  c.gamma_b = gamma_b;
  c.eos = eos < 0 ? -1 : eos;
  return dispatch(c);
}

size_t svd_cps_workspace_bytes(int64_t B, int32_t G) {
  if (B < 1 || G < 1 || G > SVD_MAX_GAMMA || B >= ((int64_t)1 << 31) / G) return 0;
  // row flags, then the records of split rows
  return align_up((size_t)B * G * sizeof(uint32_t)) + (size_t)kPartCap * sizeof(LatticePart);
}

int svd_cps_lattice(const void *q_logits, svd_dtype_t dtype, int64_t B, int32_t G, int32_t V,
                    float temp_q, float tau, int32_t m_max, int32_t eos, int32_t *cand,
                    float *cand_logp, int32_t *n_cand, int32_t *len, void *workspace,
                    size_t workspace_bytes, void *hip_stream) {
  if (!q_logits || !cand || !cand_logp || !n_cand || !len || !workspace) return SVD_EINVAL;
  if (dtype != SVD_F32 && dtype != SVD_BF16) return SVD_EDTYPE;
  if (V < 1 || !temp_ok(temp_q) || !(tau > 0.0f) || !(tau <= 1.0f) || m_max < 1 ||
      m_max > kCpsMax || eos >= V)
    return SVD_EINVAL;
  const size_t need = svd_cps_workspace_bytes(B, G);
  if (need == 0 || ((uintptr_t)workspace) % kAlign != 0) return SVD_EINVAL;
  if (workspace_bytes < need) return SVD_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  uint32_t *flags = static_cast<uint32_t *>(workspace);
  LatticePart *part = reinterpret_cast<LatticePart *>(static_cast<char *>(workspace) +
                                                      align_up((size_t)B * G * sizeof(uint32_t)));
  const float c = (float)(1.4426950408889634 / (double)temp_q);
  const size_t es = dtype == SVD_F32 ? 4 : 2;
  const bool vec = ((size_t)V * es) % 16 == 0 && ((uintptr_t)q_logits) % 16 == 0;
  const dim3 grid((unsigned)(B * G));
  const int e = eos < 0 ? -1 : eos;
  CallTimer tm;
  // few rows: slices of whole vectors, then one wave per row merges them
  const int64_t rows = B * G;
  int S = 1, slice = V;
  if (rows < kLatticeSplitRows) {
    const int unit = vec ? (int)(16 / es) : 1;
    const int64_t units = V / unit;
    const int64_t most = std::min<int64_t>(std::max<int64_t>(1, units / (2 * kSplitBlock)),
                                           kLatticeMaxSlices);
    const int64_t want = std::min<int64_t>((kSplitTarget + rows - 1) / rows, kPartCap / rows);
    const int64_t s_try = std::max<int64_t>(1, std::min(most, want));
    slice = (int)((units + s_try - 1) / s_try) * unit;
    S = (V + slice - 1) / slice;
  }
  if (S > 1) {
    const dim3 gs((unsigned)(rows * S));
    if (dtype == SVD_BF16) {
      const auto *q = static_cast<const BF16::elem *>(q_logits);
      if (vec)
        SVD_LAUNCH(tm, SVD_KERNEL_LATTICE, s, kr_lattice_split<BF16, true>, gs, dim3(kSplitBlock),
                   s, q, V, c, S, slice, part);
      else
        SVD_LAUNCH(tm, SVD_KERNEL_LATTICE, s, kr_lattice_split<BF16, false>, gs,
                   dim3(kSplitBlock), s, q, V, c, S, slice, part);
    } else {
      const auto *q = static_cast<const F32::elem *>(q_logits);
      if (vec)
        SVD_LAUNCH(tm, SVD_KERNEL_LATTICE, s, kr_lattice_split<F32, true>, gs, dim3(kSplitBlock),
                   s, q, V, c, S, slice, part);
      else
        SVD_LAUNCH(tm, SVD_KERNEL_LATTICE, s, kr_lattice_split<F32, false>, gs, dim3(kSplitBlock),
                   s, q, V, c, S, slice, part);
    }
    SVD_LAUNCH(tm, SVD_KERNEL_COMBINE, s, kr_lattice_combine,
               dim3((unsigned)((rows * 64 + kBlock - 1) / kBlock)), dim3(kBlock), s, rows, c, tau,
               m_max, e, S, (const LatticePart *)part, cand, cand_logp, n_cand, flags);
  } else if (dtype == SVD_BF16) {
    const auto *q = static_cast<const BF16::elem *>(q_logits);
    // a row of at most kLatticeRegVecs vectors per thread is held in registers
    constexpr int RB = lattice_regs<BF16, true>();
    const bool in_regs = ((int64_t)V / BF16::kPerVec + kRowBlock - 1) / kRowBlock <= RB;
    if (vec && in_regs)
      SVD_LAUNCH(tm, SVD_KERNEL_LATTICE, s, kr_lattice<BF16, true, RB>, grid, dim3(kRowBlock), s,
                 q, V, c, tau, m_max, e, cand, cand_logp, n_cand, flags);
    else if (vec)
      SVD_LAUNCH(tm, SVD_KERNEL_LATTICE, s, kr_lattice<BF16, true, 0>, grid, dim3(kRowBlock), s, q,
                 V, c, tau, m_max, e, cand, cand_logp, n_cand, flags);
    else
      SVD_LAUNCH(tm, SVD_KERNEL_LATTICE, s, kr_lattice<BF16, false, 0>, grid, dim3(kRowBlock), s,
                 q, V, c, tau, m_max, e, cand, cand_logp, n_cand, flags);
  } else {
    const auto *q = static_cast<const F32::elem *>(q_logits);
    if (vec)
      SVD_LAUNCH(tm, SVD_KERNEL_LATTICE, s, kr_lattice<F32, true, 0>, grid, dim3(kRowBlock), s, q,
                 V, c, tau, m_max, e, cand, cand_logp, n_cand, flags);
    else
      SVD_LAUNCH(tm, SVD_KERNEL_LATTICE, s, kr_lattice<F32, false, 0>, grid, dim3(kRowBlock), s, q,
                 V, c, tau, m_max, e, cand, cand_logp, n_cand, flags);
  }
  SVD_LAUNCH(tm, SVD_KERNEL_LATTICE_LEN, s, kr_lattice_len,
             dim3((unsigned)((B * 64 + kBlock - 1) / kBlock)),
             dim3(kBlock), s, (const uint32_t *)flags, B, G, m_max, cand, cand_logp, n_cand, len);
  return SVD_OK;
}

int svd_cps_beam(const int32_t *cand, const float *cand_logp, const int32_t *n_cand,
                 const int32_t *len, const float *fluency, float lambda, int64_t B, int32_t G,
                 int32_t m_max, int32_t beam, int32_t *paths, float *path_score,
                 int32_t *path_len, void *hip_stream) {
  if (!cand || !cand_logp || !n_cand || !len || !paths || !path_score || !path_len)
    return SVD_EINVAL;
  if (B < 1 || B >= ((int64_t)1 << 31) || G < 1 || G > kCpsMaxG || m_max < 1 ||
      m_max > kCpsMax || beam < 1 || beam > kCpsBeam || !std::isfinite(lambda))
    return SVD_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  CallTimer tm;
  SVD_LAUNCH(tm, SVD_KERNEL_BEAM, s, kr_cps_beam, dim3((unsigned)B), dim3(kBeamBlock), s, cand, cand_logp,
             n_cand, len, fluency, lambda, (int)G, (int)m_max, (int)beam, paths, path_score,
             path_len);
  return SVD_OK;
}

int svd_adl_next(const int32_t *drafts, const int32_t *selected, const int32_t *accept_len,
                 const int32_t *gamma_b, int32_t eos, int64_t B, int32_t K, int32_t gamma,
                 int32_t k_min, int32_t k_max, int32_t step, int32_t shift, int32_t slack,
                 int32_t *avg, int32_t *next, void *hip_stream) {
  if (!drafts || !selected || !accept_len || !avg || !next) return SVD_EINVAL;
  if (B < 1 || B >= ((int64_t)1 << 31) || K < 1 || K > SVD_MAX_K || gamma < 1 ||
      gamma > SVD_MAX_GAMMA || B >= ((int64_t)1 << 31) / ((int64_t)K * gamma))
    return SVD_EINVAL;
  if (k_min < 1 || k_max < k_min || k_max > SVD_MAX_GAMMA || step < 0 || step > SVD_MAX_GAMMA ||
      shift < 0 || shift > 16 || slack < 0 || slack > kAdlStateMax)
    return SVD_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  CallTimer tm;
  SVD_LAUNCH(tm, SVD_KERNEL_ADL, s, kr_adl, dim3((unsigned)((B + kBlock - 1) / kBlock)),
             dim3(kBlock), s, drafts, selected, accept_len, gamma_b, (int)eos, B, (int)K,
             (int)gamma, (int)k_min, (int)k_max, (int)step, (int)shift, (int)slack, avg, next);
  return SVD_OK;
}

const char *svd_strerror(int status) {
  switch (status) {
    case SVD_OK: return "success";
    case SVD_EINVAL: return "invalid argument (null pointer, size out of range, bad temperature or misaligned workspace)";
    case SVD_EDTYPE: return "unsupported logit dtype";
    case SVD_EWORKSPACE: return "workspace smaller than svd_workspace_bytes()";
    case SVD_EHIP: return "HIP kernel launch failed";
    case SVD_ESCRATCH: return "sizes need a workspace larger than the no-allocation scratch (SVD_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
