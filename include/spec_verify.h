/*
 * spec_verify.h — C ABI of the speculative-sampling verification step on MI355X (gfx950).
 *
 * The operation (defined on these pages; cited by title and section):
 *  - "Speculative Decoding : accélérer l'inférence des LLM" (blent.ai), sections
 *    "Principe et garanties mathématiques" and "Pourquoi la qualité est préservée":
 *    a drafted token x is accepted with probability min(1, p(x)/q(x)); the first rejected
 *    draft is replaced by a draw from max(p - q, 0) renormalised; a step emits between 1 and
 *    gamma + 1 tokens; at temperature zero a draft is accepted iff it is the target's argmax,
 *    which replaces it otherwise.
 *  - "Speculative Decoding — Come Accelerare l'Inferenza LLM di 2-3x" (aimpact), section
 *    "Il meccanismo": the draft hands over its distribution q for every draft step, the
 *    target yields p for every position, drafts after the first rejection are discarded.
 *  - "Speculative Decoding" (haruk1y wiki), section "数式で見る speculative decoding の正しさ":
 *    the acceptance probability alpha(x) and the correction distribution p_corr.
 *  - "Accélérer Sonar grâce à la spéculation" (Perplexity), sections "Décodage spéculatif"
 *    and "Inférence avec le décodage spéculatif": the longest acceptable prefix is kept, the
 *    target's logits at the mismatch or after the last draft are sampled for one more token,
 *    and the accepted length feeds the next step (so it stays on the device here).
 *
 * Conventions fixed by this library where the pages leave a step open:
 *  - p = softmax(z_target / T_b), q = softmax(z_draft / T_b), one temperature per request;
 *    a request is sampled iff T_b > 0, greedy otherwise (T = 0 exactly is the pages' case).
 *    Temperatures below about 1.4e-38 act as that value, and temperatures above about
 *    1.7e24 (+inf included) as that one: p is then uniform over the unmasked tokens.
 *  - uniforms[r][0] is the accept test at draft position r (accept iff u < p(x)/q(x),
 *    strictly); uniforms[r][1] is the draw for the token emitted at target row r, used only
 *    at the stop row: the residual after a rejection, or the bonus from p at row gamma_b.
 *  - The draw is an inverse CDF in vocabulary order over unnormalised weights r_k:
 *    k* = min { k : r_k > 0 and C_k > u * R }, C_k the running sum, R the total.
 *  - Greedy argmax ties resolve to the lowest index.  A draft id outside [0, V) has
 *    p(x) = q(x) = 0 and is rejected.
 *
 * Layout.  All logits are row-major with row stride V elements.  Request b has gamma_b
 * drafts; gamma_b = gamma when cu_draft is NULL (dense), else cu_draft[b+1] - cu_draft[b]
 * (CSR over draft rows, 0 <= gamma_b <= gamma).  Request b's draft rows and draft tokens
 * start at cu_draft[b] (dense: b*gamma); its target rows, uniform rows and output slots start
 * at cu_draft[b] + b (dense: b*(gamma+1)).  R_t = total target rows = R_d + B.
 *
 * Ownership.  The caller allocates and owns every buffer (device memory unless stated),
 * including the workspace.  The library allocates nothing, keeps no state between calls,
 * is reentrant for distinct workspaces, and touches only the ranges described.  Calls are
 * asynchronous on `stream` (a hipStream_t; NULL is the null stream) and never wait for the
 * device.  Two calls may share a workspace only when ordered on one stream.
 *
 * Errors.  Every entry point returns SPEC_OK (0) or a negative code; arguments are checked
 * on the host before anything is enqueued, so an argument error leaves outputs untouched.
 * SPEC_ERR_HIP means a kernel launch failed; kernels of the same call launched before it
 * stay enqueued.  Device data are not checked (that would need a sync): logits must be
 * finite or -inf (a masked entry: probability 0) with at least one finite logit per row,
 * cu_draft a valid CSR whose rows exist, uniforms in [0, 1).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

enum {
  SPEC_OK = 0,
  SPEC_ERR_NULL = -1,       /* a required pointer is NULL                                */
  SPEC_ERR_SHAPE = -2,      /* B < 0, gamma not in [0, 64], V not in [1, 2^24], a grid
                               too large, or a launch path the call cannot take          */
  SPEC_ERR_DTYPE = -3,      /* dtype is not a spec_dtype                                 */
  SPEC_ERR_WORKSPACE = -4,  /* workspace smaller than spec_verify_workspace_size, or not
                               256-byte aligned                                          */
  SPEC_ERR_HIP = -5,        /* a kernel launch failed                                    */
  SPEC_ERR_TOO_LARGE = -6   /* spec_verify_sample_static: the call's workspace would exceed
                               SPEC_STATIC_SCRATCH_BYTES                                 */
};

/* Largest gamma (drafts per request) the kernels take. */
#define SPEC_MAX_GAMMA 64

/*
 * How a verification call is launched (spec_probe.path).  Both ways compute the same step.
 *  SPEC_PATH_TWO  two launches: a row-statistics stream over every needed logit, then one that
 *                 merges, tests, sums the stop rows and draws.  Any size.
 *  SPEC_PATH_ONE  one launch, a workgroup per row tile as in the first of the two launches;
 *                 B <= 2048.  Greedy calls (spec_verify_greedy): the last tile of a request to
 *                 finish merges and writes the request's outputs.  Sampling calls: a request's
 *                 tiles meet inside the launch (device-scope atomics), claim spans of its stop
 *                 row(s), and the one completing the last span draws.  Tiles that arrive
 *                 early wait, boundedly, to help; one whose wait runs out (other work keeps
 *                 its siblings from being resident) leaves its share to the request's last
 *                 arrival, which never waits, so the results never depend on the waits.
 *                 Taken only if the call's workgroups (row slots x ceil(V / 16384)) fit in
 *                 three quarters of the device's capacity for the kernel: beyond that the
 *                 sharing would run mostly on one workgroup per request.
 *  SPEC_PATH_AUTO the library's choice, the default: one launch for calls of at most 2048 row
 *                 tiles with 16-byte aligned rows that it can take, where it measured faster
 *                 on MI355X; two launches otherwise.  Every path gives the same results.
 */
#define SPEC_PATH_AUTO 0
#define SPEC_PATH_TWO 1
#define SPEC_PATH_ONE 2

/*
 * Optional diagnostics and launch control (NULL: none, SPEC_PATH_AUTO).  Every pointer may be
 * NULL; all are device pointers except `events`.  Entries of greedy requests are written
 * only where stated.
 */
typedef struct spec_probe {
  double *p_x;        /* [R_d] p_i(x_i) at each draft position of sampled requests         */
  double *q_x;        /* [R_d] q_i(x_i)                                                    */
  float *row_max_t;   /* [R_t] max raw logit of each target row (greedy requests too)      */
  double *row_sum_t;  /* [R_t] sum_k exp((z_k - max) / T_b), sampled requests              */
  float *row_max_d;   /* [R_d] max raw logit of each draft row read (sampled requests)     */
  double *row_sum_d;  /* [R_d] as row_sum_t for draft rows                                 */
  double *resid_mass; /* [B] total probability mass of the distribution drawn from at the
                         stop row: sum_k max(p_k - q_k, 0) after a rejection, sum_k p_k
                         (= 1) for the bonus; sampled requests                            */
  void *events[8];    /* host: hipEvent_t or NULL; events[2k] / events[2k+1] are recorded by
                         the dispatch of the call's k-th kernel as it starts / ends (two
                         launches: 0 row statistics, 1 accept tests, residual and draw; one
                         launch: 0 the whole step); entries of launches not made are not
                         touched                                                        */
  int path;           /* SPEC_PATH_AUTO, _TWO or _ONE; _ONE on a call that cannot take it,
                         or another value, returns SPEC_ERR_SHAPE                         */
  unsigned int spin_limit; /* polls after which a waiting workgroup of the one-launch path
                         stops waiting and leaves its share to the last arrival (0: the
                         library's default, 2^12); a small value makes that hand-over run,
                         for tests of it; results do not depend on it                   */
} spec_probe;

/*
 * spec_verify_sample — verify gamma drafts per request and emit the step's tokens.
 *
 *  target_logits  [R_t, V] dtype   p's logits at positions 0..gamma_b of each request
 *  draft_logits   [R_d, V] dtype   q's logits at draft positions 0..gamma_b-1
 *  dtype          SPEC_F32 or SPEC_BF16, for both logit arrays
 *  draft_tokens   [R_d] int32      the drafted ids x_i
 *  uniforms       [R_t, 2] float   see the conventions above
 *  temperatures   [B] float        T_b; T_b > 0 samples, otherwise greedy (draft logits of a
 *                                  greedy request are never read)
 *  B, gamma       requests; drafts per request (dense) or the largest gamma_b (CSR)
 *  cu_draft       [B+1] int32 or NULL
 *  V              vocabulary size
 *  out_tokens     [R_t] int32      request b's slots 0..gamma_b: the n_b accepted drafts, the
 *                                  token emitted at the stop row n_b, then -1
 *  out_num_accepted [B] int32      n_b in [0, gamma_b]; the step emits n_b + 1 tokens
 *  workspace      device scratch of at least spec_verify_workspace_size(B, gamma, V, dtype)
 *                 bytes, 256-byte aligned, zero-filled before its first use; every call
 *                 leaves it ready for the next, of any shape.  Its first 512 KiB hold the
 *                 one-launch path's per-request counters (one per 128-byte line), which each
 *                 call returns to zero; the rest needs no initial contents
 *  probe          NULL, or diagnostics as above
 *  stream         hipStream_t
 *
 * B == 0 is an empty call: SPEC_OK, nothing enqueued, pointers unchecked.
 */
int spec_verify_sample(const void *target_logits, const void *draft_logits, int dtype,
                       const int32_t *draft_tokens, const float *uniforms,
                       const float *temperatures, int32_t B, int32_t gamma,
                       const int32_t *cu_draft, int64_t V, int32_t *out_tokens,
                       int32_t *out_num_accepted, void *workspace, size_t workspace_bytes,
                       const spec_probe *probe, void *stream);

/*
 * spec_verify_greedy — the temperature-zero step (blent.ai page, "Pourquoi la qualité est
 * préservée"; wiki page, "実装上の注意"): draft i is accepted iff it equals the lowest-index
 * argmax of target row i; the argmax at the stop row is emitted.  Draft logits are not
 * taken.  Arguments as for spec_verify_sample; probe fields other than row_max_t, events and
 * path are ignored.
 */
int spec_verify_greedy(const void *target_logits, int dtype, const int32_t *draft_tokens,
                       int32_t B, int32_t gamma, const int32_t *cu_draft, int64_t V,
                       int32_t *out_tokens, int32_t *out_num_accepted, void *workspace,
                       size_t workspace_bytes, const spec_probe *probe, void *stream);

/*
 * spec_verify_commit — hand a verification step's result to the next step on the device.
 *
 * "Accélérer Sonar grâce à la spéculation" (Perplexity), sections "Inférence avec le
 * décodage spéculatif" and "Planification MTP pour un jeton unique": the accepted length sets
 * the next sequence length, and a kernel that inserts the new tokens into their slots spares
 * the GPU-to-CPU synchronisation.  "Speculative Decoding : accélérer l'inférence des LLM"
 * (blent.ai), sections "Quel gain espérer ?" and "Mettre en œuvre dans vLLM": the acceptance
 * rate and the tokens per target pass are what to monitor.
 *
 *  out_tokens, out_num_accepted, cu_draft, B, gamma
 *                 a spec_verify_sample / spec_verify_greedy call's outputs and layout
 *  seq_tokens     [B, capacity] int32, row b = request b's token history (row stride capacity)
 *  seq_len        [B] int32, tokens held per row; read and updated
 *  stats          NULL, or uint64[5] accumulated (atomically) with {proposed = sum gamma_b,
 *                 accepted = sum n_b, emitted = sum (n_b + 1), requests = B, truncated};
 *                 zero it to start.  Acceptance rate = accepted / proposed, tokens per pass =
 *                 emitted / requests.
 *  accept_hist    NULL, or uint64[gamma + 1] accumulated: requests per accepted count n_b
 *  stream         hipStream_t; ordered after the verification call on the same stream
 *
 * Request b's n_b + 1 emitted tokens (slots cu_draft[b] + b .. + n_b of out_tokens) are written
 * to seq_tokens[b][seq_len[b] ..]; those at or past `capacity` are dropped and counted as
 * truncated; seq_len[b] becomes min(seq_len[b] + n_b + 1, capacity).  All pointers are device
 * pointers.  Errors: SPEC_ERR_SHAPE (B < 0, gamma outside [0, 64], capacity < 0), SPEC_ERR_NULL,
 * SPEC_ERR_HIP; B == 0 enqueues nothing.  Device data are not checked: for memory safety only,
 * a request whose n_b is negative (outside the verification's output range) is left unchanged
 * and not counted, n_b is clamped to at most gamma_b and seq_len[b] to [0, capacity].
 */
int spec_verify_commit(const int32_t *out_tokens, const int32_t *out_num_accepted,
                       const int32_t *cu_draft, int32_t B, int32_t gamma, int32_t *seq_tokens,
                       int64_t capacity, int32_t *seq_len, uint64_t *stats,
                       uint64_t *accept_hist, void *stream);

/* Longest n-gram spec_ngram_propose looks up. */
#define SPEC_NGRAM_MAX_N 64

/*
 * spec_ngram_propose — draft tokens for the next step by n-gram (prompt) lookup.
 *
 * "Speculative Decoding : accélérer l'inférence des LLM" (blent.ai), sections "N-gram lookup et
 * variantes sans modèle" and "Mettre en œuvre dans vLLM": the last n generated tokens are
 * looked up in the context and the tokens that followed them are proposed, with n between
 * prompt_lookup_min and prompt_lookup_max; no draft model.
 *
 * Conventions where the page leaves them open: request b's context is
 * seq_tokens[b][0 .. L), L = seq_len[b] (clamped to [0, capacity]); n runs from n_max down to
 * n_min, n < L; the pattern is the last n tokens; the occurrence used is the earliest start j
 * in [0, L - n) (a proper earlier occurrence, possibly overlapping the pattern); the
 * proposals are the up to gamma tokens from j + n on, stopping at L.  No occurrence for any n:
 * no proposals (a verification with gamma_b = 0 still emits one token).
 *
 *  seq_tokens   [B, capacity] int32      contexts, row stride capacity (spec_verify_commit's
 *                                        layout)
 *  seq_len      [B] int32
 *  n_min, n_max 1 <= n_min <= n_max <= SPEC_NGRAM_MAX_N
 *  gamma        proposals at most, 0..SPEC_MAX_GAMMA
 *  out_counts   [B] int32                proposals per request
 *  out_dense    [B, gamma] int32         proposals, then -1
 *  out_cu       [B + 1] int32 or NULL    prefix sums of out_counts (cu_draft of the
 *                                        verification step)
 *  out_packed   [B * gamma] int32 or NULL  proposals packed at out_cu[b] (draft_tokens of the
 *                                        verification step); NULL exactly when out_cu is
 *                                        (with gamma == 0, out_dense and out_packed may be NULL)
 *
 * All pointers are device pointers; asynchronous on `stream` (one launch, two with out_cu).
 * Errors: SPEC_ERR_SHAPE, SPEC_ERR_NULL, SPEC_ERR_HIP; B == 0 enqueues nothing.
 */
int spec_ngram_propose(const int32_t *seq_tokens, int64_t capacity, const int32_t *seq_len,
                       int32_t B, int32_t n_min, int32_t n_max, int32_t gamma,
                       int32_t *out_counts, int32_t *out_dense, int32_t *out_cu,
                       int32_t *out_packed, void *stream);

/*
 * spec_verify_sample_static — spec_verify_sample for callers that cannot allocate: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Arguments,
 * results and errors as for spec_verify_sample, without the workspace: the call uses a
 * static device array of SPEC_STATIC_SCRATCH_BYTES (16 MiB) that each device the library
 * runs on holds from the first such call until the process ends (its address is taken once
 * per device with hipGetSymbolAddress; no allocation, no memset).  A call whose
 * spec_verify_workspace_size exceeds it returns SPEC_ERR_TOO_LARGE with nothing enqueued
 * (workload sizes up to B = 512, gamma = 8, V = 128256 fit).  The array keeps the last
 * call's contents; what must start at zero (the one-launch counters) is zero at load and
 * is returned to zero by every call.  All calls on one device share the one array: calls
 * that overlap on a device (unordered streams, or other host threads) race and must not be
 * made; calls ordered on one stream are safe.
 */
#define SPEC_STATIC_SCRATCH_BYTES (16u << 20)
int spec_verify_sample_static(const void *target_logits, const void *draft_logits, int dtype,
                              const int32_t *draft_tokens, const float *uniforms,
                              const float *temperatures, int32_t B, int32_t gamma,
                              const int32_t *cu_draft, int64_t V, int32_t *out_tokens,
                              int32_t *out_num_accepted, const spec_probe *probe, void *stream);

/* Workspace bytes needed by either entry point for these sizes; 0 for invalid sizes. */
size_t spec_verify_workspace_size(int32_t B, int32_t gamma, int64_t V, int dtype);

/* Static description of a return code. */
const char *spec_verify_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
