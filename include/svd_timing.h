/*
 * svd_timing.h -- kernel timing of the timing build, libsvd_timed.so.
 *
 * libsvd_timed.so exports every entry point of svd.h, built from the same
 * sources with the same kernels and launch shapes, plus the two calls below.
 * The product library, libsvd.so, has neither call and keeps no state between
 * calls; the timing build exists for benchmarks and profiles.
 *
 * svd_profile_enable(mask) turns timing on for the kernels whose bit
 * (1 << SVD_KERNEL_*) is set in mask, and off for all with mask 0.  While it is
 * on, each entry-point call records a HIP event before and after every launch
 * of a timed kernel, on the stream that launch goes to (the events are created
 * on first use).  svd_profile_read() waits for the recorded events, adds up
 * the elapsed milliseconds per kernel into ms[0..n) (index: SVD_KERNEL_*),
 * writes the number of timed launches per kernel into launches[0..n)
 * (nullable), clears the record and returns SVD_OK; SVD_EINVAL for a NULL ms
 * or n < 0, SVD_EHIP when an event query fails.  The record is process-wide
 * and guarded by a lock, so calls on several threads are recorded whole; at
 * most 4096 calls are recorded between reads (later ones are not timed).  A
 * timing event makes the stream wait for the launch before it, so timed calls
 * run slower than untimed ones.
 */
#ifndef SVD_TIMING_H
#define SVD_TIMING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SVD_KERNEL_ROWSTATS = 0,   /* row statistics + alpha (streams every scored row pair) */
  SVD_KERNEL_SELECT = 1,     /* streak scores, argmax, first rejection                 */
  SVD_KERNEL_DRAW_PASS = 2,  /* fp64 pass over the drawn row pair                       */
  SVD_KERNEL_DRAW_PICK = 3,  /* fp64 masses and inverse CDF                             */
  SVD_KERNEL_BETA = 4,       /* optional overlap mass                                   */
  SVD_KERNEL_MARK = 5,       /* shared rows: flags of the pool rows read               */
  SVD_KERNEL_POOL_STATS = 6, /* shared rows: statistics once per pool row read          */
  SVD_KERNEL_ALPHA_ROWS = 7, /* shared rows: alpha per scored position                  */
  SVD_KERNEL_LATTICE = 8,    /* candidate lattice of the drafter rows (and its length)  */
  SVD_KERNEL_BEAM = 9,       /* beam search over the lattice                            */
  SVD_KERNEL_LATTICE_LEN = 10, /* lattice length and cleared tail                       */
  SVD_KERNEL_COMBINE = 11,   /* split rows: merge of the slices' statistics, alpha      */
  SVD_KERNEL_ROWSTATS_SPLIT = 12, /* split rows: statistics of each slice of a row pair  */
  SVD_KERNEL_ROWSTATS_LIVE = 13,  /* early exit: slices of the live prefixes' row pairs   */
  SVD_KERNEL_ADL = 14,       /* adaptive draft length: next window per prefix            */
  SVD_KERNEL_BETA_COMBINE = 15, /* split rows: beta from its slices' sums               */
  SVD_KERNEL_COUNT = 16
};

int svd_profile_enable(unsigned kernel_mask);
int svd_profile_read(double *ms, int64_t *launches, int n);

#ifdef __cplusplus
}
#endif

#endif /* SVD_TIMING_H */
