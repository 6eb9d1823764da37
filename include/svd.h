/*
 * svd.h -- C ABI of the MI355X (gfx950) library for lossless draft
 * verification with self-selection.
 *
 * The operation.  For each prefix s, K drafts of gamma tokens arrive with the
 * drafter's next-token logits q and the verifier's logits p over a vocabulary
 * of V tokens.  The verifier has scored every drafted position in one
 * parallel pass (SpecDiff-2, section 2 "Prelim: speculative decoding").  The
 * library
 *   1. takes the softmax of every verifier row and drafter row it needs, at
 *      temperatures temp_p and temp_q;
 *   2. computes the position-wise acceptance alpha_j = min(1, p(x_j)/q(x_j)),
 *      i.e. accept at once whenever q(x_j) <= p(x_j) (SpecDiff-2 section 2;
 *      the position-wise acceptance of SpecDiff-2 Figure 2);
 *   3. scores every draft by its expected accepted streak
 *      S_k = sum_{j<gamma} prod_{i<=j} alpha_{k,i} (SpecDiff-2 section 3) and
 *      keeps the argmax draft, the lowest k on an exact tie (SpecDiff-2
 *      section 5.2, self-selection by expected throughput);
 *   4. accepts the kept draft left to right while u_j < alpha_j and stops at
 *      the first rejection (SpecDiff-2 section 2; DiffuSpec section 3
 *      "Acceptance and rejection");
 *   5. draws the replacement token from the normalised residual max(0, p - q)
 *      of the rejected position (same passages), or, when all gamma tokens
 *      are accepted, a bonus token from the verifier's row gamma.
 * The committed tokens are the accepted prefix of the kept draft followed by
 * the drawn token (DiffuSpec section 3, "Accepted prefix length").
 *
 * Uniforms.  u = U(seed, row_base + b, position, purpose) with purpose 1 for
 * acceptance tests, 2 for the residual draw (position = accepted length L) and
 * 3 for the bonus draw (position = gamma).  U is the top 53 bits of
 *   KEY = SM64(SM64(SM64(SM64(seed) ^ row) ^ pos) ^ purpose)
 * times 2^-53, with SM64 the SplitMix64 output function (Steele, Lea and
 * Flood, OOPSLA 2014).  Outputs are a pure function of the inputs, seed and
 * row_base; a draw takes the first token whose cumulative weight exceeds u*Z.
 *
 * Precision.  Row statistics and alpha are computed in fp32 from exact
 * widenings of the logits; streak scores accumulate in fp64; the row pair of
 * the draw is recomputed from the logits in fp64.
 *
 * Conventions for every entry point:
 *   - Pointers to logits, drafts, outputs and the workspace are DEVICE
 *     pointers, owned by the caller; the library keeps none of them after the
 *     call returns.  Arrays are row-major and contiguous with V innermost.
 *   - Work is enqueued on hip_stream (a hipStream_t; NULL = the null stream)
 *     after the work already on it.  Nothing synchronises the host, nothing
 *     allocates device memory.  Results are valid once the stream reaches
 *     them.  Calls on different streams with different workspaces may run
 *     concurrently; calls that share a workspace must be ordered.
 *   - The return code reports only what the host can check: SVD_EINVAL for a
 *     NULL required pointer, a size below 1 or above the limits below, or a
 *     temperature that is not finite and positive or is so small (below about
 *     4.2e-39) that log2(e)/T overflows fp32; SVD_EDTYPE for an unknown
 *     dtype; SVD_EWORKSPACE for a workspace below svd_workspace_bytes();
 *     SVD_EHIP when a kernel launch fails.  Nothing is enqueued when the
 *     return code is SVD_EINVAL, SVD_EDTYPE or SVD_EWORKSPACE; after
 *     SVD_EHIP the launches before the failing one may have been enqueued.
 *   - Every flag, counter and list in the workspace is written by the
 *     call's own kernels before it is read (no memset, no host copy), so a
 *     call can be captured in a HIP graph and replayed.
 *   - Errors in the data go to the outputs: a drafted token outside [0, V),
 *     or a NaN or +inf logit, or an all -inf row, among the rows a prefix
 *     reads, sets that prefix's selected / accept_len / next_token to -1
 *     (alpha, beta and scores of that prefix are then unspecified).  -inf
 *     logits are legal and mean probability 0.
 */
#ifndef SVD_H
#define SVD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of both logit arrays (p and q share one).  The two range
 * markers give the type every int32 value, so that any value a caller passes
 * is a valid argument, rejected by the checks (SVD_EDTYPE) when it names no
 * type. */
typedef enum {
  SVD_F32 = 0,
  SVD_BF16 = 1,
  SVD_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  SVD_DTYPE_RANGE_MAX_ = 2147483647
} svd_dtype_t;

enum {
  SVD_OK = 0,
  SVD_EINVAL = -1,
  SVD_EDTYPE = -2,
  SVD_EWORKSPACE = -3,
  SVD_EHIP = -4,
  SVD_ESCRATCH = -5  /* svd_select_and_verify_noalloc: sizes need more than its scratch */
};

/* Documented limits. */
#define SVD_MAX_K 64            /* drafts per prefix                      */
#define SVD_MAX_GAMMA 4096      /* drafted positions per draft            */
/* B * K * gamma must stay below 2^31; V below 2^31. */

/*
 * Bytes of device workspace one call with these sizes needs (256-byte
 * aligned start is required).  Returns 0 for sizes the calls would reject.
 */
size_t svd_workspace_bytes(int64_t B, int32_t K, int32_t gamma, int32_t V);

/*
 * Single-draft verification: svd_select_and_verify with K = 1, bit for bit.
 *   p_logits   [B][gamma+1][V]  verifier logits; row j is p(.|s, x_<j), row
 *                               gamma is the bonus row p(.|s, x_<gamma)
 *   q_logits   [B][gamma][V]    drafter logits; row j is q(.|s, x_<j)
 *   draft      [B][gamma] int32 drafted tokens x_j
 *   accept_len [B] out          L in [0, gamma], or -1
 *   next_token [B] out          residual token (L < gamma) or bonus token
 *                               (L == gamma), or -1
 *   alpha      [B][gamma] out   nullable; fp32 alpha_j
 *   beta       [B][gamma] out   nullable; fp32 sum_v min(p_v, q_v), the
 *                               expected acceptance of position j (one
 *                               extra pass over the scored rows)
 */
int svd_verify(const void *p_logits, const void *q_logits, const int32_t *draft,
               svd_dtype_t dtype, int64_t B, int32_t gamma, int32_t V,
               float temp_p, float temp_q, uint64_t seed, uint64_t row_base,
               int32_t *accept_len, int32_t *next_token, float *alpha, float *beta,
               void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Self-selection and verification of K drafts per prefix.
 *   p_logits   [B][K][gamma+1][V]
 *   q_logits   [B][K][gamma][V]
 *   drafts     [B][K][gamma] int32
 *   selected   [B] out          kept draft k*, or -1
 *   accept_len [B] out          L of the kept draft, or -1
 *   next_token [B] out          the drawn token, or -1
 *   scores     [B][K] out       nullable; fp32 expected accepted streak S_k
 *   alpha      [B][K][gamma]    nullable
 *   beta       [B][K][gamma]    nullable
 */
int svd_select_and_verify(const void *p_logits, const void *q_logits, const int32_t *drafts,
                          svd_dtype_t dtype, int64_t B, int32_t K, int32_t gamma, int32_t V,
                          float temp_p, float temp_q, uint64_t seed, uint64_t row_base,
                          int32_t *selected, int32_t *accept_len, int32_t *next_token,
                          float *scores, float *alpha, float *beta,
                          void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Greedy acceptance (SpecDiff-2 section 5.2: the kept draft is verified
 * without its drafting probabilities, which lets drafter and verifier use
 * different tokenizers; appendix B.4: the uniform is compared with the
 * verifier probability, and a rejected token is resampled from the verifier
 * distribution with that token zeroed out).
 *
 * Same as svd_verify / svd_select_and_verify with
 *   alpha_j = p_j(x_j)                        (step 2; also the score's alpha)
 *   rejection at L: the draw is from p_L with token x_L zeroed and the rest
 *                   renormalised, i.e. the residual max(0, p - q) with q the
 *                   point mass at x_L (step 5); if nothing else has mass, p_L.
 * Selection, the acceptance test, the uniforms and the bonus draw are
 * unchanged.  No drafter logits are read, so a scored position moves one
 * logit row instead of two; temp_q does not exist.  Unlike the standard rule,
 * this one keeps the verifier's output law under any selection among the K
 * drafts.  The workspace of svd_workspace_bytes(B, K, gamma, V) suffices;
 * argument checks, data errors and outputs follow the conventions above.
 *
 *   p_logits [B][K][gamma+1][V] (svd_greedy_verify: [B][gamma+1][V])
 *   drafts   [B][K][gamma]      (svd_greedy_verify: [B][gamma])
 *   alpha    [B][K][gamma] out, nullable: p(x) in fp32
 */
int svd_greedy_verify(const void *p_logits, const int32_t *draft, svd_dtype_t dtype, int64_t B,
                      int32_t gamma, int32_t V, float temp_p, uint64_t seed, uint64_t row_base,
                      int32_t *accept_len, int32_t *next_token, float *alpha, void *workspace,
                      size_t workspace_bytes, void *hip_stream);
int svd_greedy_select_and_verify(const void *p_logits, const int32_t *drafts, svd_dtype_t dtype,
                                 int64_t B, int32_t K, int32_t gamma, int32_t V, float temp_p,
                                 uint64_t seed, uint64_t row_base, int32_t *selected,
                                 int32_t *accept_len, int32_t *next_token, float *scores,
                                 float *alpha, void *workspace, size_t workspace_bytes,
                                 void *hip_stream);

/*
 * Shared rows.  The K drafts of one diffusion pass are sampled from one set of
 * drafter marginals (SpecDiff-2 section 5.2), so their q rows can be one; and
 * drafts with a common prefix read the same verifier rows, as in the flattened
 * draft tree of SpecDiff-2 appendix B.8 (all drafts of a prefix share p row 0).
 * Here p and q are pools of rows with index tables saying which pool row each
 * scored position reads:
 *   p_rows   [n_p_rows][V]         verifier rows
 *   p_index  [B][K][gamma+1] int32 p row (b, k, j) = p_rows[p_index[b][k][j]];
 *                                  j = gamma is the bonus row
 *   q_rows   [n_q_rows][V]         drafter rows (unused, may be NULL, for
 *                                  SVD_RULE_GREEDY)
 *   q_index  [B][K][gamma] int32   q row (b, k, j) = q_rows[q_index[b][k][j]]
 *   drafts   [B][K][gamma] int32
 * The result is that of svd_select_and_verify (rule SVD_RULE_STANDARD) or
 * svd_greedy_select_and_verify (SVD_RULE_GREEDY) on the gathered dense arrays,
 * but each pool row that a scored position reads is streamed once, however
 * many positions read it.  An index outside its pool is a data error: the
 * prefix that reads it (for the bonus row: when the bonus is drawn) gets -1
 * outputs.  Limits: 1 <= n_p_rows < 2^30, 0 <= n_q_rows < 2^30 (>= 1 for the
 * standard rule); the workspace is svd_rows_workspace_bytes(B, K, gamma, V,
 * n_p_rows, n_q_rows) bytes (0 for sizes out of range).  No beta output.
 */
typedef enum {
  SVD_RULE_STANDARD = 0,
  SVD_RULE_GREEDY = 1,
  SVD_RULE_RANGE_MIN_ = -2147483647 - 1, /* any int32 is a valid argument, rejected */
  SVD_RULE_RANGE_MAX_ = 2147483647       /* (SVD_EINVAL) unless it names a rule */
} svd_rule_t;
size_t svd_rows_workspace_bytes(int64_t B, int32_t K, int32_t gamma, int32_t V,
                                int64_t n_p_rows, int64_t n_q_rows);
int svd_select_and_verify_rows(svd_rule_t rule, const void *p_rows, int64_t n_p_rows,
                               const int32_t *p_index, const void *q_rows, int64_t n_q_rows,
                               const int32_t *q_index, const int32_t *drafts, svd_dtype_t dtype,
                               int64_t B, int32_t K, int32_t gamma, int32_t V, float temp_p,
                               float temp_q, uint64_t seed, uint64_t row_base, int32_t *selected,
                               int32_t *accept_len, int32_t *next_token, float *scores,
                               float *alpha, void *workspace, size_t workspace_bytes,
                               void *hip_stream);

/*
 * Ragged, EOS-aware windows (DiffuSpec section 3, "Accepted prefix length":
 * a step commits the kept draft's accepted tokens, and an accepted EOS ends
 * the sequence with no draw; section 4.3: a controller picks each step's
 * draft length k_t, so sequences of one batch have windows of their own).
 *
 * Arrays are laid out as for svd_select_and_verify, padded to gamma.  Prefix b
 * drafts n_b = gamma_b[b] positions (gamma_b nullable: every n_b = gamma), and
 * with eos >= 0 draft k's usable positions stop at its first drafted EOS,
 * included: m_k = that length, or n_b.  Positions past m_k are not read.
 *   scores     S_k = sum_{j < m_k} prod_{i <= j} alpha_{k,i};
 *   acceptance over j < m_{k*}: L = the first rejection, or m_{k*};
 *   a fully accepted window that ends in EOS commits L tokens and draws
 *   nothing: next_token = -2;
 *   otherwise the residual draw at L < m_{k*}, or the bonus draw from p row n_b
 *   (uniform position n_b).
 * rule: SVD_RULE_STANDARD or SVD_RULE_GREEDY (q_logits may then be NULL).
 * alpha (nullable) is NaN at positions not streamed.
 * early_exit != 0 (K = 1 only, scores NULL): positions are streamed in chunks
 * and a prefix stops being streamed after the chunk that holds its first
 * rejection, which skips most rows when acceptance is low; data errors in rows
 * that are not streamed are then not detected.
 * Errors: SVD_EINVAL also for eos >= V, early_exit with K != 1 or a non-NULL
 * scores; an n_b outside [1, gamma] is a data error of prefix b (-1 outputs).
 * Workspace: svd_workspace_bytes(B, K, gamma, V).
 */
int svd_verify_window(svd_rule_t rule, const void *p_logits, const void *q_logits,
                      const int32_t *drafts, const int32_t *gamma_b, int32_t eos,
                      int32_t early_exit, svd_dtype_t dtype, int64_t B, int32_t K, int32_t gamma,
                      int32_t V, float temp_p, float temp_q, uint64_t seed, uint64_t row_base,
                      int32_t *selected, int32_t *accept_len, int32_t *next_token, float *scores,
                      float *alpha, void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Causal-consistency path search (DiffuSpec section 4.2: the diffusion
 * drafter's per-position candidates form a lattice; each position keeps its
 * candidates by cumulative probability mass, the lattice stops at the first
 * EOS, and a left-to-right beam search scores paths by drafter confidence
 * plus a causal-proxy fluency; section 5.3 settles on beam 3, M_max 15 and
 * tau 0.8).  The top paths are the drafts a call of svd_select_and_verify_rows
 * (the shared drafter rows are the marginals the lattice came from) ranks and
 * verifies.
 *
 * svd_cps_lattice: for every drafter row q_logits[B][G][V] (softmax at
 * temp_q), the tokens in order of decreasing probability (the lower index on
 * a tie) are kept until their cumulative mass reaches tau, at most m_max
 * (1..16) of them:
 *   cand      [B][G][m_max] out  candidate tokens, -1 after the kept ones
 *   cand_logp [B][G][m_max] out  their log-probabilities (natural log), -inf after
 *   n_cand    [B][G]        out  kept candidates (0 past the lattice)
 *   len       [B]           out  lattice length: the first position whose most
 *                                probable token is eos, included (that position
 *                                then keeps only eos), else G; -1 when a row
 *                                before it holds a NaN or +inf, or is all -inf
 * eos < 0: no EOS.  Workspace: svd_cps_workspace_bytes(B, G) bytes, 256-byte
 * aligned.  Probabilities are fp32; a cut at tau can differ from an exact one
 * when a running sum lies within ~1e-6 of tau.
 *
 * svd_cps_beam: a beam search of width beam (1..8) over a lattice (G <= 1024).
 * A path's score is the sum over its positions of cand_logp plus lambda times
 *   fluency [B][G][m_max][m_max] (nullable: 0)  the causal proxy's score of
 *   candidate i at position j after candidate a at position j-1 (a = 0 at
 *   j = 0: after the context),
 * computed in fp64.  Every step keeps the beam best expansions (path rank, then
 * candidate rank order breaks exact ties).  Outputs, best first:
 *   paths      [B][beam][G] out  tokens, -1 padded
 *   path_score [B][beam]    out  -inf for a missing path
 *   path_len   [B][beam]    out  len[b], or 0 for a missing path
 * A prefix with len[b] outside [1, G] or an n_cand outside [1, m_max] before
 * len[b] gets no paths.
 */
size_t svd_cps_workspace_bytes(int64_t B, int32_t G);
int svd_cps_lattice(const void *q_logits, svd_dtype_t dtype, int64_t B, int32_t G, int32_t V,
                    float temp_q, float tau, int32_t m_max, int32_t eos, int32_t *cand,
                    float *cand_logp, int32_t *n_cand, int32_t *len, void *workspace,
                    size_t workspace_bytes, void *hip_stream);
int svd_cps_beam(const int32_t *cand, const float *cand_logp, const int32_t *n_cand,
                 const int32_t *len, const float *fluency, float lambda, int64_t B, int32_t G,
                 int32_t m_max, int32_t beam, int32_t *paths, float *path_score,
                 int32_t *path_len, void *hip_stream);

/*
 * Adaptive draft length (DiffuSpec section 4.3, "Adaptive Draft Length": the
 * controller sets each sequence's next draft length k_t from the EOS-aware
 * generated length and the accepted length; it expands the window while
 * acceptance keeps pace with generation on average and stops expanding once
 * the generated length saturates).  Run after svd_verify_window (or any
 * select-and-verify call) on its inputs and outputs; `next` can be the next
 * call's gamma_b directly, with no trip to the host.  Per prefix b:
 *   n   = gamma_b[b] (gamma_b nullable: gamma) is this step's window, and
 *   g   = the generated length of the kept draft k = selected[b]: through its
 *         first drafted eos among positions < n (eos >= 0), else n;
 *   avg [B][2] int32 in/out holds {A, G}, the recent accepted and generated
 *         lengths in 1/256ths of a token (start them at 256 * the first window);
 *         each moves toward this step's 256 * L (L = accept_len[b]) and 256 * g
 *         by 2^-shift of the gap, rounded down;
 *   next[b] = n              when g < n (the draft ended at EOS inside the
 *                            window: the generated length has saturated),
 *             n + step       else when A + slack >= G (acceptance keeps pace),
 *             min(n, ceil(A / 256) + 1) otherwise (acceptance lags: the recent
 *                            streak plus the position that is rejected),
 *           clamped to [k_min, k_max].
 *   A prefix whose selected or accept_len is -1 (or out of range) keeps its
 *   window and state; a window outside [1, gamma] or a state outside
 *   [0, 2^20] gives next[b] = -1 and leaves the state.
 *   drafts [B][K][gamma] int32 as given to the verification call.
 * Errors (SVD_EINVAL, nothing enqueued): a NULL pointer other than gamma_b;
 * B, K or gamma out of the limits above; not 1 <= k_min <= k_max <= 4096;
 * step outside [0, 4096]; shift outside [0, 16]; slack outside [0, 2^20].
 * No workspace.
 */
int svd_adl_next(const int32_t *drafts, const int32_t *selected, const int32_t *accept_len,
                 const int32_t *gamma_b, int32_t eos, int64_t B, int32_t K, int32_t gamma,
                 int32_t k_min, int32_t k_max, int32_t step, int32_t shift, int32_t slack,
                 int32_t *avg, int32_t *next, void *hip_stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * operation, arguments and outputs as svd_select_and_verify (bit for bit), but
 * no workspace argument: the workspace is a device array of
 * SVD_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, allocated when
 * the library's code is loaded on that GPU and held until the process ends.
 * The call itself allocates and frees nothing; its first call on a device
 * looks up the array's address there (hipGetSymbolAddress), with that device
 * current, so hip_stream must belong to the current device.
 *   - SVD_ESCRATCH when svd_workspace_bytes(B, K, gamma, V) exceeds
 *     SVD_NOALLOC_SCRATCH_BYTES (16 MiB: at gamma = 8 and V = 152064, up to
 *     about 1000 prefixes); every argument error as for svd_select_and_verify;
 *     all of them before any HIP call.  SVD_EHIP when the array's address
 *     cannot be found.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents; each call writes every part it reads before reading it.
 *     Calls that overlap on one GPU (on different streams, or from different
 *     threads without ordering) race on the array: order them.
 */
#define SVD_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int svd_select_and_verify_noalloc(const void *p_logits, const void *q_logits,
                                  const int32_t *drafts, svd_dtype_t dtype, int64_t B, int32_t K,
                                  int32_t gamma, int32_t V, float temp_p, float temp_q,
                                  uint64_t seed, uint64_t row_base, int32_t *selected,
                                  int32_t *accept_len, int32_t *next_token, float *scores,
                                  float *alpha, float *beta, void *hip_stream);

/* Static text for a status code. */
const char *svd_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* SVD_H */
