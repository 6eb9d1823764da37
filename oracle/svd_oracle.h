/*
 * svd_oracle.h -- plain double-precision CPU oracle for lossless draft
 * verification with self-selection.
 *
 * TEST INFRASTRUCTURE ONLY.  This oracle exists to check the GPU library.
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load it.  It shares no source, header, table or helper with
 * the HIP library, and the library never calls it.
 *
 * What it computes (sources are the SpecDiff-2 and DiffuSpec pages):
 *   - softmax of every verifier row p(.|s,x_<j) and drafter row q(.|s,x_<j)
 *     (SpecDiff-2, section 2 "Prelim: speculative decoding": both models expose
 *     next-token posteriors; the verifier scores all positions in parallel);
 *   - the position-wise acceptance alpha_j = min(1, p(x_j)/q(x_j)), written as
 *     "accept at once when q <= p" (SpecDiff-2 section 2);
 *   - the expected accepted streak sum_j prod_{i<=j} alpha_i of every draft
 *     (SpecDiff-2 section 3 and Figure 2: alpha_j is the chance that token j is
 *     accepted once the first j-1 were) and the argmax draft (SpecDiff-2
 *     section 5.2, self-selection: keep the draft of greatest expected
 *     throughput);
 *   - left-to-right acceptance against counter-hash uniforms, stopping at the
 *     first rejection (SpecDiff-2 section 2; DiffuSpec section 3 "Acceptance
 *     and rejection");
 *   - the replacement token from the normalised residual max(0, p - q)
 *     (same passages), or a bonus token from verifier row gamma when every
 *     drafted token is accepted.
 *
 * Every logit is widened exactly to double, every step runs in double, and
 * every sum runs sequentially in vocabulary order.
 */
#ifndef SVD_ORACLE_H
#define SVD_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of the logit arrays */
enum { SVDO_F32 = 0, SVDO_BF16 = 1 };

/* SplitMix64 output function (Steele, Lea and Flood, OOPSLA 2014). */
uint64_t svdo_splitmix64(uint64_t x);
/* KEY = SM64(SM64(SM64(SM64(seed) ^ row) ^ pos) ^ purpose) */
uint64_t svdo_key(uint64_t seed, uint64_t row, uint64_t pos, uint64_t purpose);
/* U = (KEY >> 11) * 2^-53, a double in [0, 1) */
double svdo_uniform(uint64_t seed, uint64_t row, uint64_t pos, uint64_t purpose);

/* Softmax of one row at temperature T.  prob[v] = exp(z_v/T - m) / S.
 * Returns 1 for a valid row, 0 when the row holds a NaN or +inf, or is all
 * -inf (prob is then left unspecified). */
int svdo_softmax_row(const void *row, int dtype, int32_t V, float T, double *prob);

/* Inverse CDF over non-negative weights r[0..V): the first v whose running sum
 * (sequential, index order) exceeds t; if none does, the last v with r_v > 0;
 * -1 if every weight is zero.  *c_lo and *c_hi (nullable) receive the running
 * sum just before and just after the chosen index. */
int32_t svdo_inverse_cdf(const double *r, int32_t V, double t, double *c_lo, double *c_hi);

/* The distribution a draw is taken from, written into r[0..V): the residual
 * max(0, p - q) for a rejection, or p itself when q is NULL (the bonus draw)
 * or when the residual has no mass.  Returns Z = sum of r (sequential). */
double svdo_draw_weights(const double *p, const double *q, int32_t V, double *r);

/* Per-prefix diagnostics used by the parity harness to recognise near-ties. */
typedef struct {
  double select_gap;   /* S_best - S_second (+inf when K == 1)                    */
  double emit_margin;  /* min(t - C_lo, C_hi - t) / Z at the emitted token         */
  double draw_z;       /* Z of the draw                                             */
  double draw_t;       /* t = u * Z                                                 */
} svdo_diag_t;

/*
 * Full verification of B prefixes.
 *   p_logits [B][K][gamma+1][V], q_logits [B][K][gamma][V], drafts [B][K][gamma].
 *   force_k / force_L (nullable, per prefix, -1 = not forced) pin the selected
 *   draft and / or the accepted length, so that a harness can re-run the later
 *   steps conditioned on another implementation's earlier decision.
 * Outputs (all nullable except selected, accept_len, next_token):
 *   scores [B][K]; alpha, beta, px, qx [B][K][gamma];
 *   accept_margin [B][gamma] = |u_j - alpha_{k*,j}| for every j;
 *   diag [B].
 * A prefix whose inputs are invalid gets -1 in selected, accept_len, next_token.
 * nthreads >= 1 worker threads split the prefixes.  Returns 0, or -1 on bad
 * arguments.
 */
int svdo_select_and_verify(const void *p_logits, const void *q_logits, const int32_t *drafts,
                           int dtype, int64_t B, int32_t K, int32_t gamma, int32_t V,
                           float temp_p, float temp_q, uint64_t seed, uint64_t row_base,
                           const int32_t *force_k, const int32_t *force_L,
                           int32_t *selected, int32_t *accept_len, int32_t *next_token,
                           double *scores, double *alpha, double *beta, double *px, double *qx,
                           double *accept_margin, svdo_diag_t *diag, int nthreads);

/*
 * Greedy acceptance (SpecDiff-2 section 5.2: the kept draft is verified
 * without its drafting probabilities; appendix B.4: the uniform is compared
 * with the verifier probability, and a rejected token is resampled from the
 * verifier distribution with that token zeroed).  alpha_{k,j} = p_j(x_{k,j});
 * scores, selection, acceptance and the bonus draw as above; the rejection
 * draw is the residual max(0, p - q) with q the point mass at the rejected
 * token.  p_logits and drafts as above; no drafter rows.  alpha and px
 * receive the same values.
 */
int svdo_greedy_select_and_verify(const void *p_logits, const int32_t *drafts, int dtype,
                                  int64_t B, int32_t K, int32_t gamma, int32_t V, float temp_p,
                                  uint64_t seed, uint64_t row_base, const int32_t *force_k,
                                  const int32_t *force_L, int32_t *selected, int32_t *accept_len,
                                  int32_t *next_token, double *scores, double *alpha,
                                  double *accept_margin, svdo_diag_t *diag, int nthreads);

/*
 * Ragged, EOS-aware windows (DiffuSpec section 3, "Accepted prefix length":
 * a step commits the kept draft's accepted tokens, and an accepted EOS ends
 * the sequence with no draw; section 4.3: k_t is chosen anew every step).
 * Prefix b drafts n = gamma_b[b] positions (1 <= n <= gamma; NULL: gamma) in
 * arrays padded to gamma.  With eos >= 0, draft k's usable length m_k stops at
 * its first drafted EOS, included (else m_k = n).  Then
 *   score      S_k = sum_{j < m_k} prod_{i <= j} alpha_{k,i};
 *   acceptance over j < m_{k*}: L = the first rejection, or m_{k*};
 *   an accepted window ending in EOS commits L tokens and draws nothing
 *   (next_token = -2); otherwise the residual draw at L < m_{k*}, or the bonus
 *   draw from p row n with uniform position n.
 * Rows past m_k are never read and their alpha is not written.  An n outside
 * [1, gamma] invalidates the prefix.  greedy: the greedy-acceptance rule (no
 * q_logits).  Returns 0, or -1 on bad arguments.
 */
int svdo_window_select_and_verify(int greedy, const void *p_logits, const void *q_logits,
                                  const int32_t *drafts, const int32_t *gamma_b, int32_t eos,
                                  int dtype, int64_t B, int32_t K, int32_t gamma, int32_t V,
                                  float temp_p, float temp_q, uint64_t seed, uint64_t row_base,
                                  const int32_t *force_k, const int32_t *force_L,
                                  int32_t *selected, int32_t *accept_len, int32_t *next_token,
                                  double *scores, double *alpha, double *accept_margin,
                                  svdo_diag_t *diag, int nthreads);

/*
 * Causal-consistency path search (DiffuSpec section 4.2; settings in section
 * 5.3).  svdo_cps_lattice: for each drafter row q_logits[b][j] (softmax at
 * temp_q), the tokens in order of decreasing logit (lower index on a tie) are
 * kept until their cumulative probability reaches tau, at most m_max of them:
 * cand[b][j][0..n_cand), cand_logp = their log-probabilities, -1 / -inf after.
 * The lattice of prefix b stops at the first position whose most probable
 * token is EOS, which is then that position's only candidate: len[b] = that
 * position + 1, else G (-1 for an invalid row).  cum_margin (nullable): the
 * distance of the last two cumulative sums from tau.
 * svdo_cps_beam: a left-to-right beam search of width `beam` over the lattice.
 * A path's score is the sum over its positions of cand_logp plus lambda times
 * fluency[b][j][a][i], the causal proxy's score of candidate i at position j
 * after candidate a at position j - 1 (a = 0 at j = 0: after the context);
 * fluency may be NULL (0).  Each step keeps the `beam` best expansions, the
 * earlier one (path rank, then candidate rank) on an exact tie.  Outputs:
 * paths[b][beam][G] tokens (-1 padded), path_score, path_len (0 for a missing
 * path), rank_margin[b] = the smallest score gap between consecutive kept
 * expansions, or between the last kept and the best dropped one.
 */
int svdo_cps_lattice(const void *q_logits, int dtype, int64_t B, int32_t G, int32_t V,
                     float temp_q, double tau, int32_t m_max, int32_t eos, int32_t *cand,
                     double *cand_logp, int32_t *n_cand, int32_t *len, double *cum_margin);
int svdo_cps_beam(const int32_t *cand, const double *cand_logp, const int32_t *n_cand,
                  const int32_t *len, const float *fluency, double lambda, int64_t B, int32_t G,
                  int32_t m_max, int32_t beam, int32_t *paths, double *path_score,
                  int32_t *path_len, double *rank_margin);

/*
 * Adaptive draft length (DiffuSpec section 4.3, "Adaptive Draft Length"): the
 * next step's window of every sequence, from this step's accepted length and
 * EOS-aware generated length, read as follows.  Per prefix b:
 *   n  = gamma_b[b] (NULL: gamma), this step's window; outside [1, gamma]:
 *        a data error (next[b] = -1, state unchanged);
 *   k  = selected[b], L = accept_len[b]; either negative (a prefix whose
 *        inputs were invalid): next[b] = n, state unchanged;
 *   g  = the generated length of draft k: its first eos at j < n gives j + 1,
 *        else n (eos < 0: n);
 *   the state avg[b] = {A, G} holds the recent accepted and generated lengths
 *   in 1/256ths of a token, each moved toward this step's value by 2^-shift
 *   of the gap, rounded down:  A += floor((256 L - A) / 2^shift), the same
 *   for G with g; a state outside [0, 2^20] is a data error (-1, unchanged);
 *   then
 *     g < n (the draft ended at EOS inside the window: the generated length
 *            has saturated)                   next = n              (hold)
 *     A + slack >= G (acceptance keeps pace with generation, on average)
 *                                              next = n + step       (expand)
 *     otherwise                                next = ceil(A / 256) + 1, at
 *                                              most n                (shrink)
 *   and next is clamped to [k_min, k_max].
 * Returns 0, or -1 for parameters out of range (1 <= k_min <= k_max <= 4096,
 * 0 <= step <= 4096, 0 <= shift <= 16, 0 <= slack <= 2^20, 1 <= gamma <= 4096,
 * 1 <= K <= 64).
 */
int svdo_adl_next(const int32_t *drafts, const int32_t *selected, const int32_t *accept_len,
                  const int32_t *gamma_b, int32_t eos, int64_t B, int32_t K, int32_t gamma,
                  int32_t k_min, int32_t k_max, int32_t step, int32_t shift, int32_t slack,
                  int32_t *avg, int32_t *next);

#ifdef __cplusplus
}
#endif

#endif /* SVD_ORACLE_H */
