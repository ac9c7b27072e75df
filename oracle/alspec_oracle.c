/*
 * CPU oracle for the speculative flash-decode step of attention-level
 * speculation (ALSpec).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, double-precision
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header, table or helper with the GPU library, and the GPU
 * library never loads it.
 *
 * Sources (web pages on the method):
 *   [P1] "Attention-Level Speculation", atlas.scime.ai research-map summary:
 *        sections "Summary", "Approach", "Key results", "Limitations".
 *   [P2] "Attention-Level Speculation", ICML 2025 poster page: abstract.
 *
 * What the pages fix, restated: each layer's self-attention output is
 * speculated with a cheap attention-sink approximation; exact attention is
 * computed as well; the approximation is checked against the exact output
 * with a relative L2 threshold (lambda = 0.10 in the evaluation) and is then
 * committed or discarded ([P1] Summary, Approach, Key results; [P2]
 * abstract).  The pages' evaluation checked the outcome in simulation,
 * with the approximate and the exact attention both evaluated ([P1]
 * Limitations); this oracle likewise computes both.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - the sink approximation is softmax attention restricted to the first S
 *     tokens and the last W tokens of the context, renormalised over that set
 *     (the attention-sink construction of "Efficient Streaming Language
 *     Models with Attention Sinks", which the pages cite by title);
 *   - the sets are sink = [0, min(S,L)), window = [max(min(S,L), L-W), L);
 *     they never overlap;
 *   - the relative L2 error is taken per (user, layer) over the
 *     concatenated [Hq x D] attention output before any output projection;
 *   - commit iff ratio <= lambda; a NaN ratio never commits; a zero exact
 *     output gives ratio 0 when the difference is also zero, else +inf;
 *   - query head h reads kv head h / (Hq / Hkv) (contiguous GQA groups);
 *   - logits are sm_scale * <q, k>.
 *
 * Arithmetic: double throughout.  fp32 inputs are widened exactly; bf16
 * inputs (raw 16-bit patterns) are widened exactly by placing them in the
 * high half of an IEEE binary32 word.  Softmax is the two-pass textbook form
 * (max, then exp and sums) over the whole set, with no splitting.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

/* ---- exact widening of the stored key/value element types -------------- */

static double widen_f32(const void *base, size_t idx) {
  return (double)((const float *)base)[idx];
}

static double widen_bf16(const void *base, size_t idx) {
  uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

typedef double (*widen_fn)(const void *, size_t);

/* ---- one query head over an explicit list of token positions ----------- */

/*
 * Softmax attention state of one query vector over the token positions in
 * `tok` (any order, no repeats): m = max logit, l = sum exp(s - m),
 * acc[d] = sum exp(s - m) * v[d].  An empty list gives m = -inf, l = 0,
 * acc = 0.  This is the per-split state that flash decoding keeps (the
 * pages name flash decoding as a building block: [P1] "Builds on").
 */
static void head_state(int D, widen_fn wk, const void *k, const void *v,
                       size_t row0, const float *q, const int32_t *tok,
                       int ntok, double sm_scale, double *s_buf, double *m_out,
                       double *l_out, double *acc) {
  double m = -INFINITY;
  for (int t = 0; t < ntok; ++t) {
    size_t row = row0 + (size_t)tok[t] * (size_t)D;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += (double)q[d] * wk(k, row + (size_t)d);
    double s = sm_scale * dot;
    s_buf[t] = s;
    if (s > m) m = s;
  }
  double l = 0.0;
  for (int d = 0; d < D; ++d) acc[d] = 0.0;
  for (int t = 0; t < ntok; ++t) {
    size_t row = row0 + (size_t)tok[t] * (size_t)D;
    double w = exp(s_buf[t] - m);
    l += w;
    for (int d = 0; d < D; ++d) acc[d] += w * wk(v, row + (size_t)d);
  }
  *m_out = m;
  *l_out = l;
}

/* ---- the token sets of the approximation -------------------------------- */

/* sink = [0, s_end), window = [w_begin, L), middle = [s_end, w_begin). */
static void token_sets(int L, int S, int W, int *s_end, int *w_begin) {
  int se = S < L ? S : L;
  int wb = L - W;
  if (wb < se) wb = se;
  *s_end = se;
  *w_begin = wb;
}

/* ---- exact and approximate attention for every (user, query head) ------ */

typedef struct {
  int B, Hq, Hkv, D, L_cap, S, W;
  const int32_t *seq_lens;
  widen_fn wk;
  const float *q;
  const void *k, *v;
  double sm_scale;
  double *o_exact, *lse_exact, *o_approx, *lse_approx, *mass_A;
  int next_pair, npairs, nthreads;
  int failed;
} job_t;

typedef struct {
  job_t *job;
  int tid;
} worker_arg_t;

static void one_pair(job_t *J, int pair, int32_t *tok_all, int32_t *tok_A,
                     double *s_buf, double *acc_e, double *acc_a) {
  int b = pair / J->Hq, h = pair % J->Hq;
  int G = J->Hq / J->Hkv;
  int g = h / G;
  int L = J->seq_lens[b];
  int D = J->D;
  size_t row0 = ((size_t)b * J->Hkv + g) * (size_t)J->L_cap * (size_t)D;
  const float *qh = J->q + ((size_t)b * J->Hq + h) * (size_t)D;

  int s_end, w_begin;
  token_sets(L, J->S, J->W, &s_end, &w_begin);
  int nA = 0;
  for (int j = 0; j < L; ++j) tok_all[j] = j;
  for (int j = 0; j < s_end; ++j) tok_A[nA++] = j;
  for (int j = w_begin; j < L; ++j) tok_A[nA++] = j;

  double m_e, l_e, m_a, l_a;
  head_state(D, J->wk, J->k, J->v, row0, qh, tok_all, L, J->sm_scale, s_buf,
             &m_e, &l_e, acc_e);
  head_state(D, J->wk, J->k, J->v, row0, qh, tok_A, nA, J->sm_scale, s_buf,
             &m_a, &l_a, acc_a);

  size_t o = ((size_t)b * J->Hq + h) * (size_t)D;
  for (int d = 0; d < D; ++d) {
    J->o_exact[o + d] = acc_e[d] / l_e;
    J->o_approx[o + d] = acc_a[d] / l_a;
  }
  size_t bh = (size_t)b * J->Hq + h;
  if (J->lse_exact) J->lse_exact[bh] = m_e + log(l_e);
  if (J->lse_approx) J->lse_approx[bh] = m_a + log(l_a);
  /* exact softmax mass that falls on the approximation set */
  if (J->mass_A) J->mass_A[bh] = l_a * exp(m_a - m_e) / l_e;
}

static void *worker(void *argp) {
  worker_arg_t *a = (worker_arg_t *)argp;
  job_t *J = a->job;
  int Lmax = J->L_cap;
  int32_t *tok_all = (int32_t *)malloc(sizeof(int32_t) * (size_t)(Lmax + 1));
  int32_t *tok_A = (int32_t *)malloc(sizeof(int32_t) * (size_t)(Lmax + 1));
  double *s_buf = (double *)malloc(sizeof(double) * (size_t)(Lmax + 1));
  double *acc_e = (double *)malloc(sizeof(double) * (size_t)J->D);
  double *acc_a = (double *)malloc(sizeof(double) * (size_t)J->D);
  if (!tok_all || !tok_A || !s_buf || !acc_e || !acc_a) {
    J->failed = 1;
  } else {
    /* static round-robin assignment: pair p goes to thread p % nthreads */
    for (int p = a->tid; p < J->npairs; p += J->nthreads)
      one_pair(J, p, tok_all, tok_A, s_buf, acc_e, acc_a);
  }
  free(tok_all);
  free(tok_A);
  free(s_buf);
  free(acc_e);
  free(acc_a);
  return NULL;
}

/*
 * Relative L2 test of [P1] Summary / Approach (threshold value from [P1] Key
 * results), per batch entry b over the n = Hq*D outputs of that entry:
 *   num = sum (o_approx - o_exact)^2, den = sum o_exact^2,
 *   ratio = sqrt(num / den), commit = (ratio <= lambda).
 */
int oracle_verify(int B, int n, const double *o_approx, const double *o_exact,
                  double lambda, double *ratio, uint8_t *commit) {
  if (B < 0 || n <= 0 || !o_approx || !o_exact || !ratio || !commit)
    return ORACLE_EINVAL;
  for (int b = 0; b < B; ++b) {
    double num = 0.0, den = 0.0;
    for (int i = 0; i < n; ++i) {
      double e = o_exact[(size_t)b * n + i];
      double diff = o_approx[(size_t)b * n + i] - e;
      num += diff * diff;
      den += e * e;
    }
    double r;
    if (isnan(num) || isnan(den))
      r = NAN;
    else if (den > 0.0)
      r = sqrt(num / den);
    else
      r = (num == 0.0) ? 0.0 : INFINITY;
    ratio[b] = r;
    commit[b] = (uint8_t)(r <= lambda); /* false for NaN */
  }
  return ORACLE_OK;
}

/*
 * The whole step for B batch entries (one (user, layer) each):
 *   q  : fp32 [B][Hq][D]
 *   k,v: fp32 or bf16 bit patterns, [B][Hkv][L_cap][D]
 *   outputs (double): o_exact, o_approx, o_committed [B][Hq][D];
 *   lse_exact, lse_approx, mass_A [B][Hq] (each may be NULL);
 *   ratio [B], commit [B].
 * Returns 0, or ORACLE_EINVAL / ORACLE_ENOMEM.
 */
int oracle_spec_decode(int B, int Hq, int Hkv, int D, int L_cap,
                       const int32_t *seq_lens, int kv_bf16, const float *q,
                       const void *k, const void *v, int S, int W,
                       double sm_scale, double lambda, int nthreads,
                       double *o_exact, double *lse_exact, double *o_approx,
                       double *lse_approx, double *mass_A, double *ratio,
                       uint8_t *commit, double *o_committed) {
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || L_cap < 1 || Hq % Hkv != 0)
    return ORACLE_EINVAL;
  if (!seq_lens || !q || !k || !v || !o_exact || !o_approx || !ratio ||
      !commit || !o_committed)
    return ORACLE_EINVAL;
  if (S < 0 || W < 0 || S + W < 1 || !(lambda >= 0.0) || !(sm_scale > 0.0))
    return ORACLE_EINVAL;
  for (int b = 0; b < B; ++b)
    if (seq_lens[b] < 1 || seq_lens[b] > L_cap) return ORACLE_EINVAL;
  if (nthreads < 1) nthreads = 1;

  job_t J;
  memset(&J, 0, sizeof J);
  J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.D = D; J.L_cap = L_cap; J.S = S; J.W = W;
  J.seq_lens = seq_lens;
  J.wk = kv_bf16 ? widen_bf16 : widen_f32;
  J.q = q; J.k = k; J.v = v;
  J.sm_scale = sm_scale;
  J.o_exact = o_exact; J.lse_exact = lse_exact;
  J.o_approx = o_approx; J.lse_approx = lse_approx; J.mass_A = mass_A;
  J.npairs = B * Hq;
  if (nthreads > J.npairs) nthreads = J.npairs;
  J.nthreads = nthreads;

  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  worker_arg_t *args =
      (worker_arg_t *)malloc(sizeof(worker_arg_t) * (size_t)nthreads);
  if (!th || !args) {
    free(th);
    free(args);
    return ORACLE_ENOMEM;
  }
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    args[t].job = &J;
    args[t].tid = t;
    if (t == 0) continue; /* thread 0 is the caller */
    if (pthread_create(&th[t], NULL, worker, &args[t]) != 0) {
      args[t].tid = -1; /* run its share below */
    } else {
      ++started;
    }
  }
  worker(&args[0]);
  for (int t = 1; t < nthreads; ++t) {
    if (args[t].tid < 0) {
      args[t].tid = t;
      worker(&args[t]);
    } else {
      pthread_join(th[t], NULL);
    }
  }
  (void)started;
  free(th);
  free(args);
  if (J.failed) return ORACLE_ENOMEM;

  int n = Hq * D;
  int rc = oracle_verify(B, n, o_approx, o_exact, lambda, ratio, commit);
  if (rc) return rc;
  /* committed output: the approximation on commit, exact attention otherwise
     ([P1] Approach: commit or discard) */
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < n; ++i) {
      size_t x = (size_t)b * n + i;
      o_committed[x] = commit[b] ? o_approx[x] : o_exact[x];
    }
  return ORACLE_OK;
}

/*
 * State (m, l, acc[D]) of one query head over the listed token positions of
 * one kv head (q_head: fp32 [D]; k_head, v_head: [L_cap][D] of the stored
 * type).  Positions must lie in [0, L_cap).
 */
int oracle_partial(int D, int L_cap, int kv_bf16, const float *q_head,
                   const void *k_head, const void *v_head,
                   const int32_t *tokens, int ntok, double sm_scale,
                   double *m, double *l, double *acc) {
  if (D < 1 || L_cap < 1 || ntok < 0 || !q_head || !k_head || !v_head || !m ||
      !l || !acc || (ntok > 0 && !tokens))
    return ORACLE_EINVAL;
  for (int t = 0; t < ntok; ++t)
    if (tokens[t] < 0 || tokens[t] >= L_cap) return ORACLE_EINVAL;
  double *s_buf = (double *)malloc(sizeof(double) * (size_t)(ntok + 1));
  if (!s_buf) return ORACLE_ENOMEM;
  head_state(D, kv_bf16 ? widen_bf16 : widen_f32, k_head, v_head, 0, q_head,
             tokens, ntok, sm_scale, s_buf, m, l, acc);
  free(s_buf);
  return ORACLE_OK;
}

/*
 * Log-sum-exp merge of n partial states (m_i, l_i, acc_i[D]) into one
 * normalised output, as flash decoding combines its splits:
 *   M = max m_i;  Z = sum l_i e^(m_i - M);  out = sum acc_i e^(m_i - M) / Z;
 *   lse = M + ln Z.
 * States with m_i = -inf (empty splits) carry no weight.  Returns
 * ORACLE_EINVAL when every state is empty.
 */
int oracle_lse_merge(int n, int D, const double *m, const double *l,
                     const double *acc, double *out, double *lse) {
  if (n < 1 || D < 1 || !m || !l || !acc || !out) return ORACLE_EINVAL;
  double M = -INFINITY;
  for (int i = 0; i < n; ++i)
    if (m[i] > M) M = m[i];
  if (M == -INFINITY) return ORACLE_EINVAL;
  double Z = 0.0;
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  for (int i = 0; i < n; ++i) {
    if (m[i] == -INFINITY) continue;
    double w = exp(m[i] - M);
    Z += l[i] * w;
    for (int d = 0; d < D; ++d) out[d] += acc[(size_t)i * D + d] * w;
  }
  for (int d = 0; d < D; ++d) out[d] /= Z;
  if (lse) *lse = M + log(Z);
  return ORACLE_OK;
}
