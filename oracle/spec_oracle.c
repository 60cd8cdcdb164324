/*
 * Plain fp64 CPU oracle for the speculative-sampling verification step.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this file's library.  It shares no code, header, table or constant with the
 * HIP library: it is written from the method's definition and is deliberately slow and
 * literal (no blocking, no fusion, one request at a time; OpenMP only hands whole requests
 * to threads, which leaves every request's arithmetic unchanged).
 *
 * What it follows (the pages' titles; sections in brackets):
 *  - "Speculative Decoding : accélérer l'inférence des LLM" (blent.ai) [Principe et
 *    garanties mathématiques; Pourquoi la qualité est préservée]: the draft proposes gamma
 *    tokens, the target scores every position in one pass; a drafted token x is accepted
 *    with probability min(1, p(x)/q(x)); on rejection the replacement is drawn from
 *    max(p - q, 0) renormalised; at least one and at most gamma + 1 tokens are emitted;
 *    at temperature zero a token is accepted iff it equals the target's argmax, and the
 *    argmax replaces it otherwise.
 *  - "Speculative Decoding — Come Accelerare l'Inferenza LLM di 2-3x" (aimpact) [Il
 *    meccanismo]: q is kept for every draft step, p comes for every position, the drafts
 *    after the first rejection are discarded.
 *  - "Speculative Decoding" (haruk1y wiki) [数式で見る speculative decoding の正しさ]:
 *    alpha(x) = min(1, p(x)/q(x)) and p_corr(x) = max(p(x)-q(x),0) / sum max(p-q,0).
 *  - "Accélérer Sonar grâce à la spéculation" (Perplexity) [Décodage spéculatif]: the
 *    longest acceptable prefix is kept and the target's logits at the mismatch, or after
 *    the last draft, are sampled for one more token.
 *
 * Readings taken where the pages leave a step open (all stated again with the tests):
 *  - p = softmax(z_target / T), q = softmax(z_draft / T), the same T for both; a request
 *    is sampled iff T > 0 and greedy otherwise.
 *  - Uniform pair per target row: [i][0] is the accept test at draft position i (accept iff
 *    u < p(x)/q(x), strictly); [i][1] is the draw for the token emitted at row i, used only
 *    at the stop row (residual after a rejection, or the bonus from p at row gamma_b).
 *  - Inverse CDF in index order over the unnormalised weights r_k:
 *    k* = min { k : r_k > 0 and C_k > u * R } with C_k the running sum and R = C_{V-1}.
 *  - q(x) = 0 gives ratio +inf if p(x) > 0 and 0 if p(x) = 0; a draft id outside [0, V)
 *    has p(x) = q(x) = 0 and is rejected.
 *  - If the residual mass is zero (impossible in exact arithmetic), sample from p instead
 *    and count a fallback.
 *  - Argmax ties resolve to the lowest index (+0.0 and -0.0 compare equal).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1 };

/* One stored logit as an exact double. bf16 is the upper half of an IEEE binary32. */
static double logit_at(const void *base, int dtype, int64_t idx) {
  if (dtype == OR_F32) return (double)((const float *)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Row maximum and lowest index attaining it. */
static void row_argmax(const void *base, int dtype, int64_t row, int64_t V,
                       double *max_out, int64_t *idx_out) {
  double best = logit_at(base, dtype, row * V);
  int64_t bi = 0;
  for (int64_t k = 1; k < V; ++k) {
    double z = logit_at(base, dtype, row * V + k);
    if (z > best) { best = z; bi = k; }
  }
  *max_out = best;
  *idx_out = bi;
}

/* Unnormalised softmax weight exp((z - m) / T) of a logit z in a row whose maximum is m.  A
 * masked logit (-inf) has weight 0 at every temperature: written out, because at T = +inf the
 * quotient (-inf - m) / T is not a number. */
static double weight(double z, double m, double T) {
  if (z == -INFINITY) return 0.0;
  return exp((z - m) / T);
}

/* Softmax normaliser at temperature T: m = max_k z_k, S = sum_k exp((z_k - m) / T); a row
 * needs one finite logit. */
static void row_softmax_stats(const void *base, int dtype, int64_t row, int64_t V, double T,
                              double *m_out, double *S_out) {
  double m;
  int64_t unused;
  row_argmax(base, dtype, row, V, &m, &unused);
  double S = 0.0;
  for (int64_t k = 0; k < V; ++k) S += weight(logit_at(base, dtype, row * V + k), m, T);
  *m_out = m;
  *S_out = S;
}

/* p_k = exp((z_k - m) / T) / S */
static double prob(const void *base, int dtype, int64_t row, int64_t V, double T, double m,
                   double S, int64_t k) {
  return weight(logit_at(base, dtype, row * V + k), m, T) / S;
}

typedef struct {
  double *p_x, *q_x, *margin;      /* [R_d] */
  double *row_max_t, *row_sum_t;   /* [R_t] */
  double *row_max_d, *row_sum_d;   /* [R_d] */
  double *resid_mass, *cdf_gap;    /* [B]   */
  int32_t *fallback;               /* [B]   */
} diag_t;

/*
 * Inverse-CDF draw over weights r_0..r_{V-1} >= 0 given by `weight(k)`.
 * Returns k* and writes R and the CDF gap in u units.
 */
typedef double (*weight_fn)(void *ctx, int64_t k);

static int64_t inverse_cdf(weight_fn weight, void *ctx, int64_t V, double u, double *R_out,
                           double *gap_out) {
  double R = 0.0;
  for (int64_t k = 0; k < V; ++k) R += weight(ctx, k);
  *R_out = R;
  double target = u * R;
  double C = 0.0, C_prev = 0.0;
  int64_t last_pos = -1;
  for (int64_t k = 0; k < V; ++k) {
    double r = weight(ctx, k);
    C_prev = C;
    C += r;
    if (r > 0.0) {
      last_pos = k;
      if (C > target) {
        double g1 = u - C_prev / R, g2 = C / R - u;
        *gap_out = g1 < g2 ? g1 : g2;
        return k;
      }
    }
  }
  /* Reached only for u >= 1 or a rounding corner: the last token with positive weight. */
  *gap_out = 0.0;
  return last_pos < 0 ? 0 : last_pos;
}

typedef struct {
  const void *t, *d;
  int dtype;
  int64_t trow, drow, V;
  double T, mt, St, md, Sd;
} resid_ctx;

static double resid_weight(void *vctx, int64_t k) {
  resid_ctx *c = (resid_ctx *)vctx;
  double p = prob(c->t, c->dtype, c->trow, c->V, c->T, c->mt, c->St, k);
  double q = prob(c->d, c->dtype, c->drow, c->V, c->T, c->md, c->Sd, k);
  return p > q ? p - q : 0.0;
}

static double target_weight(void *vctx, int64_t k) {
  resid_ctx *c = (resid_ctx *)vctx;
  return prob(c->t, c->dtype, c->trow, c->V, c->T, c->mt, c->St, k);
}

static void verify_one(const void *target, const void *draft, int dtype,
                       const int32_t *draft_tokens, const float *uniforms,
                       const float *temperatures, int32_t B, int32_t gamma,
                       const int32_t *cu_draft, int64_t V, int32_t b, int32_t *out_tokens,
                       int32_t *out_num_accepted, const diag_t *dg) {
  (void)B;
  int64_t dbase = cu_draft ? cu_draft[b] : (int64_t)b * gamma;
  int64_t gb = cu_draft ? (int64_t)cu_draft[b + 1] - cu_draft[b] : gamma;
  int64_t tbase = dbase + b;
  double T = temperatures ? (double)temperatures[b] : 0.0;
  int64_t n = gb;        /* accepted count */
  int64_t emitted = -1;  /* the token emitted at row n */

  if (!(T > 0.0)) {
    /* Greedy: accept while the draft equals the target argmax; emit the argmax at the stop. */
    for (int64_t i = 0; i <= gb; ++i) {
      double mx;
      int64_t g;
      row_argmax(target, dtype, tbase + i, V, &mx, &g);
      if (dg->row_max_t) dg->row_max_t[tbase + i] = mx;
      if (i == gb) { emitted = g; break; }
      if ((int64_t)draft_tokens[dbase + i] != g) { n = i; emitted = g; break; }
    }
  } else {
    /* Row statistics of every target and draft row of the request. */
    double *mt = (double *)malloc(sizeof(double) * (size_t)(gb + 1));
    double *St = (double *)malloc(sizeof(double) * (size_t)(gb + 1));
    double *md = (double *)malloc(sizeof(double) * (size_t)(gb > 0 ? gb : 1));
    double *Sd = (double *)malloc(sizeof(double) * (size_t)(gb > 0 ? gb : 1));
    for (int64_t i = 0; i <= gb; ++i) {
      row_softmax_stats(target, dtype, tbase + i, V, T, &mt[i], &St[i]);
      if (dg->row_max_t) dg->row_max_t[tbase + i] = mt[i];
      if (dg->row_sum_t) dg->row_sum_t[tbase + i] = St[i];
    }
    for (int64_t i = 0; i < gb; ++i) {
      row_softmax_stats(draft, dtype, dbase + i, V, T, &md[i], &Sd[i]);
      if (dg->row_max_d) dg->row_max_d[dbase + i] = md[i];
      if (dg->row_sum_d) dg->row_sum_d[dbase + i] = Sd[i];
    }
    /* Sequential accept test; the first rejection ends the accepted prefix. */
    for (int64_t i = 0; i < gb; ++i) {
      int64_t x = draft_tokens[dbase + i];
      double p = 0.0, q = 0.0;
      if (x >= 0 && x < V) {
        p = prob(target, dtype, tbase + i, V, T, mt[i], St[i], x);
        q = prob(draft, dtype, dbase + i, V, T, md[i], Sd[i], x);
      }
      double ratio = q > 0.0 ? p / q : (p > 0.0 ? INFINITY : 0.0);
      double u = (double)uniforms[2 * (tbase + i) + 0];
      if (dg->p_x) dg->p_x[dbase + i] = p;
      if (dg->q_x) dg->q_x[dbase + i] = q;
      if (n == gb) {  /* still inside the accepted prefix: this decision counts */
        if (dg->margin) dg->margin[dbase + i] = fabs(u - ratio);
        if (!(u < ratio)) n = i;
      }
    }
    /* The token at the stop row: residual after a rejection, bonus from p otherwise. */
    resid_ctx c = {target, draft, dtype, tbase + n, dbase + n, V, T, mt[n], St[n],
                   n < gb ? md[n] : 0.0, n < gb ? Sd[n] : 1.0};
    double u = (double)uniforms[2 * (tbase + n) + 1];
    double R = 0.0, gap = 0.0;
    int32_t fb = 0;
    if (n < gb) {
      emitted = inverse_cdf(resid_weight, &c, V, u, &R, &gap);
      if (!(R > 0.0)) {
        fb = 1;
        emitted = inverse_cdf(target_weight, &c, V, u, &R, &gap);
      }
    } else {
      emitted = inverse_cdf(target_weight, &c, V, u, &R, &gap);
    }
    if (dg->resid_mass) dg->resid_mass[b] = R;
    if (dg->cdf_gap) dg->cdf_gap[b] = gap;
    if (dg->fallback) dg->fallback[b] = fb;
    free(mt); free(St); free(md); free(Sd);
  }

  for (int64_t i = 0; i <= gb; ++i) {
    int32_t v;
    if (i < n) v = draft_tokens[dbase + i];
    else if (i == n) v = (int32_t)emitted;
    else v = -1;
    out_tokens[tbase + i] = v;
  }
  out_num_accepted[b] = (int32_t)n;
}

/*
 * Verify the requests listed in `requests` (all B when NULL).  `temperatures == NULL`
 * means every request is greedy and `draft` is never read.  Layout as in the library:
 * dense (cu_draft == NULL): request b's draft rows start at b*gamma, its target rows, uniform
 * rows and output slots at b*(gamma+1); ragged: draft rows at cu_draft[b], the others at
 * cu_draft[b] + b.  Every diagnostic pointer may be NULL.  Returns 0, or -1 on bad sizes.
 */
int oracle_verify(const void *target, const void *draft, int dtype,
                  const int32_t *draft_tokens, const float *uniforms,
                  const float *temperatures, int32_t B, int32_t gamma,
                  const int32_t *cu_draft, int64_t V, const int32_t *requests,
                  int32_t n_requests, int32_t *out_tokens, int32_t *out_num_accepted,
                  double *p_x, double *q_x, double *margin, double *row_max_t,
                  double *row_sum_t, double *row_max_d, double *row_sum_d,
                  double *resid_mass, double *cdf_gap, int32_t *fallback, int num_threads) {
  if (B < 0 || V < 1 || (dtype != OR_F32 && dtype != OR_BF16)) return -1;
  diag_t dg = {p_x, q_x, margin, row_max_t, row_sum_t, row_max_d, row_sum_d,
               resid_mass, cdf_gap, fallback};
  int32_t count = requests ? n_requests : B;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int32_t k = 0; k < count; ++k) {
    int32_t b = requests ? requests[k] : k;
    verify_one(target, draft, dtype, draft_tokens, uniforms, temperatures, B, gamma,
               cu_draft, V, b, out_tokens, out_num_accepted, &dg);
  }
  return 0;
}

/*
 * After a verification step, commit each request's emitted tokens to its token history and
 * count what the step did.
 *
 * Follows "Accélérer Sonar grâce à la spéculation" (Perplexity) [Inférence avec le décodage
 * spéculatif; Planification MTP pour un jeton unique]: the accepted length sets the next
 * sequence length, and instead of a GPU-to-CPU synchronisation a kernel inserts the next
 * tokens into their slots.  The counters follow "Speculative Decoding : accélérer l'inférence
 * des LLM" (blent.ai) [Quel gain espérer ?; Mettre en œuvre dans vLLM]: the acceptance rate
 * and the tokens produced per target pass are the quantities to monitor.
 *
 * Readings: request b's history is row b of `seq_tokens` (row stride `capacity`), holding
 * seq_len[b] tokens.  The step emitted out_tokens[t_b .. t_b + n_b] (n_b accepted drafts, then
 * the drawn token), t_b = cu_draft[b] + b (dense: b (gamma + 1)).  They are written at
 * positions seq_len[b] .. seq_len[b] + n_b; positions at or past `capacity` are not written
 * and count as truncated; the new length is min(seq_len[b] + n_b + 1, capacity).  stats (may
 * be NULL) accumulates {proposed = sum gamma_b, accepted = sum n_b, emitted = sum (n_b + 1),
 * requests = B, truncated}; hist (may be NULL, gamma + 1 bins) counts requests by n_b.
 * Returns 0, or -1 (nothing written) on bad sizes or an accepted count outside [0, gamma_b] (a
 * verification step accepts between 0 and gamma_b drafts).
 */
int oracle_commit(const int32_t *out_tokens, const int32_t *num_accepted,
                  const int32_t *cu_draft, int32_t B, int32_t gamma, int32_t *seq_tokens,
                  int64_t capacity, int32_t *seq_len, uint64_t *stats, uint64_t *hist) {
  if (B < 0 || gamma < 0 || capacity < 0) return -1;
  for (int32_t b = 0; b < B; ++b) {  /* every count checked before anything is written */
    int64_t gb = cu_draft ? (int64_t)cu_draft[b + 1] - cu_draft[b] : gamma;
    if (gb < 0 || gb > gamma || num_accepted[b] < 0 || num_accepted[b] > gb) return -1;
  }
  for (int32_t b = 0; b < B; ++b) {
    int64_t dbase = cu_draft ? cu_draft[b] : (int64_t)b * gamma;
    int64_t gb = cu_draft ? (int64_t)cu_draft[b + 1] - cu_draft[b] : gamma;
    int64_t tbase = dbase + b;
    int64_t n = num_accepted[b];
    int64_t len = seq_len[b];
    uint64_t lost = 0;
    for (int64_t i = 0; i <= n; ++i) {
      int64_t pos = len + i;
      if (pos < capacity) seq_tokens[b * capacity + pos] = out_tokens[tbase + i];
      else lost++;
    }
    seq_len[b] = (int32_t)(len + n + 1 < capacity ? len + n + 1 : capacity);
    if (stats) {
      stats[0] += (uint64_t)gb;
      stats[1] += (uint64_t)n;
      stats[2] += (uint64_t)(n + 1);
      stats[3] += 1;
      stats[4] += lost;
    }
    if (hist) hist[n] += 1;
  }
  return 0;
}

/*
 * N-gram (prompt lookup) drafting for the next step.
 *
 * Follows "Speculative Decoding : accélérer l'inférence des LLM" (blent.ai) [N-gram lookup et
 * variantes sans modèle; Mettre en œuvre dans vLLM]: the last n generated tokens are looked
 * up in the context and the tokens that followed them there are proposed as drafts, with n
 * bounded by prompt_lookup_min and prompt_lookup_max; no model is involved.
 *
 * Readings (the page leaves them open): request b's context is h = seq_tokens[b][0 .. L),
 * L = seq_len[b].  n runs from n_max down to n_min (longest first), n < L; the pattern is the
 * suffix h[L-n .. L); the occurrence used is the earliest j in [0, L - n) with
 * h[j .. j+n) == h[L-n .. L) (a proper earlier occurrence; it may overlap the suffix); the
 * proposals are h[j+n .. min(j+n+gamma, L)), at least one token.  The first n with an
 * occurrence decides; with none, the request gets no proposals.
 * Outputs: counts[b]; dense[b][0 .. gamma) (proposals then -1); when cu is not NULL,
 * cu[0..B] = prefix sums of counts and packed[cu[b] ..] = request b's proposals (the draft
 * layout of the verification step); match_j / match_n (may be NULL): j and n, or -1 and 0.
 * Returns 0, or -1 on bad sizes.
 */
int oracle_ngram(const int32_t *seq_tokens, int64_t capacity, const int32_t *seq_len,
                 int32_t B, int32_t n_min, int32_t n_max, int32_t gamma, int32_t *counts,
                 int32_t *dense, int32_t *cu, int32_t *packed, int32_t *match_j,
                 int32_t *match_n) {
  if (B < 0 || capacity < 0 || n_min < 1 || n_max < n_min || gamma < 0) return -1;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t *h = seq_tokens + (int64_t)b * capacity;
    int64_t L = seq_len[b];
    if (L < 0) L = 0;
    if (L > capacity) L = capacity;
    int64_t found_j = -1, found_n = 0;
    for (int64_t n = n_max; n >= n_min && found_j < 0; --n) {
      if (n >= L) continue;
      for (int64_t j = 0; j < L - n; ++j) {
        int64_t k = 0;
        while (k < n && h[j + k] == h[L - n + k]) ++k;
        if (k == n) {
          found_j = j;
          found_n = n;
          break;
        }
      }
    }
    int64_t cnt = 0;
    if (found_j >= 0) {
      int64_t start = found_j + found_n;
      cnt = L - start < gamma ? L - start : gamma;
    }
    counts[b] = (int32_t)cnt;
    for (int64_t i = 0; i < gamma; ++i)
      dense[(int64_t)b * gamma + i] = i < cnt ? h[found_j + found_n + i] : -1;
    if (match_j) match_j[b] = (int32_t)found_j;
    if (match_n) match_n[b] = (int32_t)found_n;
  }
  if (cu) {
    cu[0] = 0;
    for (int32_t b = 0; b < B; ++b) cu[b + 1] = cu[b] + counts[b];
    if (packed)
      for (int32_t b = 0; b < B; ++b)
        for (int32_t i = 0; i < counts[b]; ++i) packed[cu[b] + i] = dense[(int64_t)b * gamma + i];
  }
  return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
