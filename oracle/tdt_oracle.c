/*
 * TEST INFRASTRUCTURE ONLY — plain CPU float64 oracle for the Token-and-Duration
 * Transducer (TDT) loss, forward and backward.
 *
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The GPU path never calls it and shares no code with it.
 *
 * What it computes follows the description of the kernels on the page
 * "tdt-loss: add TDT loss kernel" (huggingface/kernels-community PR #882, comment
 * "What's in it"): a log-softmax over the vocabulary of every lattice node, a
 * log-softmax over the duration logits, float64 alpha/beta passes over the lattice,
 * gradients with respect to the token and the duration logits, and the reductions
 * mean_volume, mean_batch, mean, sum and none.  The pages give no equations; the
 * transition rules below are the plain reading that the rest supports (blank moves
 * advance the frame index by a positive duration, label moves advance the label
 * index by one with any allowed duration including 0, sigma is subtracted once from
 * the token log-probability of every emission, a path ends only when a blank lands
 * exactly on t = T at u = U).
 *
 * Everything is float64 in the log domain, with plain loops and no blocking or
 * reordering beyond what the definition states.  Inputs stored as fp32, fp16 or
 * bf16 are widened exactly to float64 element by element.
 *
 * Notation for one utterance b: T = logit_lengths[b], U = label_lengths[b],
 * labels y_1..y_U, nodes n = (t, u) with 0 <= t < T and 0 <= u <= U, token logits
 * h(n) in R^V, duration logits g(n) in R^D, durations d_0..d_{D-1}.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_F16 1
#define ORACLE_BF16 2
#define ORACLE_F64 3 /* float64 logits: used only to pin the oracle by finite differences */

#define RED_NONE 0
#define RED_SUM 1
#define RED_MEAN 2
#define RED_MEAN_BATCH 3
#define RED_MEAN_VOLUME 4

/* per-utterance status bits (same meaning as documented in the test helpers) */
#define ST_BAD_LOGIT_LENGTH 1
#define ST_BAD_LABEL_LENGTH 2
#define ST_BAD_LABEL 4
#define ST_INFEASIBLE 8

/* ---- exact widening of the stored element types to float64 ---- */

static double half_bits_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 0x1f;
  int man = h & 0x3ff;
  double v;
  if (ex == 0) {
    v = ldexp((double)man, -24); /* subnormal: man * 2^-24 */
  } else if (ex == 31) {
    v = man ? NAN : INFINITY;
  } else {
    v = ldexp((double)(man + 1024), ex - 25); /* (1.man) * 2^(ex-15) */
  }
  return sign ? -v : v;
}

static double bf16_bits_to_double(uint16_t h) {
  uint32_t bits = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double load_elem(int dtype, const void* base, int64_t off) {
  if (dtype == ORACLE_F32) return (double)((const float*)base)[off];
  if (dtype == ORACLE_F16) return half_bits_to_double(((const uint16_t*)base)[off]);
  if (dtype == ORACLE_F64) return ((const double*)base)[off];
  return bf16_bits_to_double(((const uint16_t*)base)[off]);
}

/* log(sum_i exp(x_i)) with the maximum factored out; -inf for an empty or all -inf set. */
static double log_sum_exp(const double* x, int n) {
  double m = -INFINITY;
  for (int i = 0; i < n; ++i)
    if (x[i] > m) m = x[i];
  if (m == -INFINITY) return -INFINITY;
  if (isnan(m)) return NAN;
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += exp(x[i] - m);
  return m + log(s);
}

typedef struct {
  int dtype;
  int64_t B, Tmax, U1max, V, D;
  const void* tok;
  int64_t ts0, ts1, ts2;
  const void* dur;
  int64_t ds0, ds1, ds2;
  const int64_t* labels;
  int64_t lab_stride;
  const int64_t* Tlen;
  const int64_t* Ulen;
  const int32_t* durations;
  int32_t blank;
  double sigma;
} problem_t;

static int64_t node_index(const problem_t* p, int64_t b, int64_t t, int64_t u) {
  return (b * p->Tmax + t) * p->U1max + u;
}

/* Status of utterance b before any arithmetic: lengths within the padded shapes and
 * labels inside the vocabulary. */
static int utterance_status(const problem_t* p, int64_t b) {
  int64_t T = p->Tlen[b], U = p->Ulen[b];
  int st = 0;
  if (T < 0 || T > p->Tmax) st |= ST_BAD_LOGIT_LENGTH;
  if (U < 0 || U > p->U1max - 1) st |= ST_BAD_LABEL_LENGTH;
  if (!(st & ST_BAD_LABEL_LENGTH)) {
    for (int64_t u = 0; u < U; ++u) {
      int64_t y = p->labels[b * p->lab_stride + u];
      if (y < 0 || y >= p->V) st |= ST_BAD_LABEL;
    }
  }
  return st;
}

/*
 * Per-utterance working set.  lp_blank[t][u] = log softmax(h(t,u))[blank],
 * lp_label[t][u] = log softmax(h(t,u))[y_{u+1}] (u < U), lam[t][u][i] =
 * log softmax(g(t,u))[i], lse_h / lse_g the two log-normalisers.
 */
typedef struct {
  int64_t T, U;
  double* lse_h;
  double* lse_g;
  double* lp_blank;
  double* lp_label;
  double* lam;
  double* alpha;
  double* beta;
  double logp_alpha, logp_beta;
} utt_t;

#define AT(arr, t, u) ((arr)[(t) * (U + 1) + (u)])

/* Step 1: log-softmax over the V token logits and over the D duration logits of each node. */
static void node_log_probs(const problem_t* p, int64_t b, utt_t* w) {
  const int64_t T = w->T, U = w->U, V = p->V, D = p->D;
  int64_t nn = T * (U + 1);
#pragma omp parallel
  {
    double* buf = (double*)malloc(sizeof(double) * (size_t)(V > D ? V : D));
#pragma omp for schedule(static)
    for (int64_t idx = 0; idx < nn; ++idx) {
      int64_t t = idx / (U + 1), u = idx % (U + 1);
      const int64_t base = b * p->ts0 + t * p->ts1 + u * p->ts2;
      for (int64_t v = 0; v < V; ++v) buf[v] = load_elem(p->dtype, p->tok, base + v);
      double lh = log_sum_exp(buf, (int)V);
      w->lse_h[idx] = lh;
      w->lp_blank[idx] = buf[p->blank] - lh;
      if (u < U) {
        int64_t y = p->labels[b * p->lab_stride + u];
        w->lp_label[idx] = buf[y] - lh;
      } else {
        w->lp_label[idx] = -INFINITY;
      }
      const int64_t dbase = b * p->ds0 + t * p->ds1 + u * p->ds2;
      for (int64_t i = 0; i < D; ++i) buf[i] = load_elem(p->dtype, p->dur, dbase + i);
      double lg = log_sum_exp(buf, (int)D);
      w->lse_g[idx] = lg;
      for (int64_t i = 0; i < D; ++i) w->lam[idx * D + i] = buf[i] - lg;
    }
    free(buf);
  }
}

/* log-weight of the blank move with duration index i out of node (t,u) */
static double blank_weight(const problem_t* p, const utt_t* w, int64_t t, int64_t u, int64_t i) {
  const int64_t U = w->U;
  return AT(w->lp_blank, t, u) - p->sigma + w->lam[(t * (U + 1) + u) * p->D + i];
}

/* log-weight of the label move with duration index i out of node (t,u), u < U */
static double label_weight(const problem_t* p, const utt_t* w, int64_t t, int64_t u, int64_t i) {
  const int64_t U = w->U;
  return AT(w->lp_label, t, u) - p->sigma + w->lam[(t * (U + 1) + u) * p->D + i];
}

/* Steps 2-4: alpha(0,0) = 0; alpha(n) = log-sum-exp over every move e into n of
 * alpha(source) + weight(e).  logP_alpha collects the blank moves that land on t = T
 * from u = U. */
static void forward_alpha(const problem_t* p, utt_t* w) {
  const int64_t T = w->T, U = w->U, D = p->D;
  double* terms = (double*)malloc(sizeof(double) * (size_t)(2 * D + 1));
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t u = 0; u <= U; ++u) {
      if (t == 0 && u == 0) {
        AT(w->alpha, t, u) = 0.0;
        continue;
      }
      int n = 0;
      for (int64_t i = 0; i < D; ++i) {
        int64_t d = p->durations[i];
        if (d > 0 && t - d >= 0) /* blank from (t-d, u) */
          terms[n++] = AT(w->alpha, t - d, u) + blank_weight(p, w, t - d, u, i);
        if (u >= 1 && t - d >= 0) /* label y_u from (t-d, u-1) */
          terms[n++] = AT(w->alpha, t - d, u - 1) + label_weight(p, w, t - d, u - 1, i);
      }
      AT(w->alpha, t, u) = log_sum_exp(terms, n);
    }
  }
  int n = 0;
  for (int64_t i = 0; i < D; ++i) {
    int64_t d = p->durations[i];
    if (d > 0 && T - d >= 0) terms[n++] = AT(w->alpha, T - d, U) + blank_weight(p, w, T - d, U, i);
  }
  w->logp_alpha = log_sum_exp(terms, n);
  free(terms);
}

/* Step 5: beta(n) = log-sum-exp over every move e out of n of weight(e) + beta(dest),
 * where the terminal has beta = 0.  logP_beta = beta(0,0). */
static void backward_beta(const problem_t* p, utt_t* w) {
  const int64_t T = w->T, U = w->U, D = p->D;
  double* terms = (double*)malloc(sizeof(double) * (size_t)(2 * D + 1));
  for (int64_t t = T - 1; t >= 0; --t) {
    for (int64_t u = U; u >= 0; --u) {
      int n = 0;
      for (int64_t i = 0; i < D; ++i) {
        int64_t d = p->durations[i];
        if (d > 0) {
          if (t + d < T)
            terms[n++] = blank_weight(p, w, t, u, i) + AT(w->beta, t + d, u);
          else if (t + d == T && u == U)
            terms[n++] = blank_weight(p, w, t, u, i);
        }
        if (u < U && t + d < T) terms[n++] = label_weight(p, w, t, u, i) + AT(w->beta, t + d, u + 1);
      }
      AT(w->beta, t, u) = log_sum_exp(terms, n);
    }
  }
  w->logp_beta = T > 0 ? AT(w->beta, 0, 0) : -INFINITY;
  free(terms);
}

typedef struct {
  /* optional per-node outputs, indexed by (b*Tmax + t)*U1max + u; NULL to skip */
  double* lse_h;
  double* lse_g;
  double* alpha;
  double* beta;
  double* occ;    /* O(n) = posterior probability that a path leaves n */
  double* cblank; /* posterior expected number of blank moves out of n */
  double* clabel; /* posterior expected number of label moves out of n */
  double* cdur;   /* [.][D] posterior expected number of moves of duration index i out of n */
} node_out_t;

/* Posteriors of the moves out of every node of one utterance, indexed by t*(U+1) + u. */
typedef struct {
  double* occ;  /* O(n) = exp(alpha(n) + beta(n) - log P) */
  double* cb;   /* c_blank(n): sum of the posteriors of the blank moves out of n */
  double* cl;   /* c_label(n): sum of the posteriors of the label moves out of n */
  double* cdur; /* [.][D] c_dur(n, i): sum of the posteriors of the moves of duration index i */
} post_t;

/*
 * Step 7: the posterior of a move e out of n is exp(alpha(n) + weight(e) + beta(dest) - log P)
 * (beta of the terminal = 0); O(n), c_blank(n), c_label(n) and c_dur(n, i) are the sums
 * named above.
 */
static post_t node_posteriors(const problem_t* p, const utt_t* w, double logP) {
  const int64_t T = w->T, U = w->U, D = p->D;
  const int64_t nn = T * (U + 1);
  post_t q;
  q.cdur = (double*)calloc((size_t)(nn * D > 0 ? nn * D : 1), sizeof(double));
  q.cb = (double*)calloc((size_t)(nn > 0 ? nn : 1), sizeof(double));
  q.cl = (double*)calloc((size_t)(nn > 0 ? nn : 1), sizeof(double));
  q.occ = (double*)calloc((size_t)(nn > 0 ? nn : 1), sizeof(double));
#pragma omp parallel for schedule(static)
  for (int64_t idx = 0; idx < nn; ++idx) {
    int64_t t = idx / (U + 1), u = idx % (U + 1);
    double a = w->alpha[idx];
    double cb = 0.0, cl = 0.0;
    for (int64_t i = 0; i < D; ++i) {
      int64_t d = p->durations[i];
      double gi = 0.0;
      if (d > 0) {
        double lb = -INFINITY;
        if (t + d < T)
          lb = AT(w->beta, t + d, u);
        else if (t + d == T && u == U)
          lb = 0.0;
        if (lb != -INFINITY) {
          double g = exp(a + blank_weight(p, w, t, u, i) + lb - logP);
          cb += g;
          gi += g;
        }
      }
      if (u < U && t + d < T) {
        double g = exp(a + label_weight(p, w, t, u, i) + AT(w->beta, t + d, u + 1) - logP);
        cl += g;
        gi += g;
      }
      q.cdur[idx * D + i] = gi;
    }
    q.cb[idx] = cb;
    q.cl[idx] = cl;
    q.occ[idx] = exp(a + w->beta[idx] - logP);
  }
  return q;
}

static void free_posteriors(post_t* q) {
  free(q->cdur);
  free(q->cb);
  free(q->cl);
  free(q->occ);
}

/*
 * Step 8 and the reduction weight, for one node (t, u) of utterance b:
 *   orow_t[v] = wb * (O(n) softmax(h(n))_v - [v = blank] c_blank(n) - [v = y_{u+1}] c_label(n))
 *   orow_d[i] = wb * (O(n) softmax(g(n))_i - c_dur(n, i))
 * Either output may be NULL.
 */
static void gradient_row(const problem_t* p, int64_t b, const utt_t* w, const post_t* q, int64_t t, int64_t u,
                         double wb, double* orow_t, double* orow_d) {
  const int64_t U = w->U, V = p->V, D = p->D;
  int64_t idx = t * (U + 1) + u;
  double O = q->occ[idx];
  const int64_t base = b * p->ts0 + t * p->ts1 + u * p->ts2;
  if (orow_t) {
    double lh = w->lse_h[idx];
    for (int64_t v = 0; v < V; ++v) {
      double hv = load_elem(p->dtype, p->tok, base + v);
      orow_t[v] = O * exp(hv - lh);
    }
    orow_t[p->blank] -= q->cb[idx];
    if (u < U) orow_t[p->labels[b * p->lab_stride + u]] -= q->cl[idx];
    for (int64_t v = 0; v < V; ++v) orow_t[v] *= wb;
  }
  if (orow_d) {
    for (int64_t i = 0; i < D; ++i) orow_d[i] = wb * (O * exp(w->lam[idx * D + i]) - q->cdur[idx * D + i]);
  }
}

/*
 * Steps 7-8 for utterance b: the node posteriors go to the per-node outputs; the gradient
 * rows (scaled by the reduction weight wb) go to the full gradient when gtok / gdur are
 * not NULL, and to rtok / rdur for the selected padded node indices `rows` of this
 * utterance.
 */
static void node_posteriors_and_grads(const problem_t* p, int64_t b, const utt_t* w, double logP, double wb,
                                      const node_out_t* no, double* gtok, double* gdur, const int64_t* rows,
                                      int64_t nrows, double* rtok, double* rdur) {
  const int64_t T = w->T, U = w->U, V = p->V, D = p->D;
  const int64_t nn = T * (U + 1);
  post_t q = node_posteriors(p, w, logP);
  if (no) {
    for (int64_t idx = 0; idx < nn; ++idx) {
      int64_t t = idx / (U + 1), u = idx % (U + 1);
      int64_t n = node_index(p, b, t, u);
      if (no->lse_h) no->lse_h[n] = w->lse_h[idx];
      if (no->lse_g) no->lse_g[n] = w->lse_g[idx];
      if (no->alpha) no->alpha[n] = w->alpha[idx];
      if (no->beta) no->beta[n] = w->beta[idx];
      if (no->occ) no->occ[n] = q.occ[idx];
      if (no->cblank) no->cblank[n] = q.cb[idx];
      if (no->clabel) no->clabel[n] = q.cl[idx];
      if (no->cdur)
        for (int64_t i = 0; i < D; ++i) no->cdur[n * D + i] = q.cdur[idx * D + i];
    }
  }
  /* gradient rows: full tensor and/or a list of selected nodes of this utterance */
  const int64_t per_b = p->Tmax * p->U1max;
  if (gtok || gdur) {
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t j = 0; j < nn; ++j) {
      int64_t t = j / (U + 1), u = j % (U + 1);
      int64_t n = node_index(p, b, t, u);
      gradient_row(p, b, w, &q, t, u, wb, gtok ? gtok + n * V : NULL, gdur ? gdur + n * D : NULL);
    }
  }
  if (rows) {
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t j = 0; j < nrows; ++j) {
      int64_t n = rows[j];
      if (n / per_b != b) continue;
      int64_t t = (n / p->U1max) % p->Tmax;
      int64_t u = n % p->U1max;
      if (t >= T || u > U) continue; /* padding: the caller zero-filled it */
      gradient_row(p, b, w, &q, t, u, wb, rtok ? rtok + j * V : NULL, rdur ? rdur + j * D : NULL);
    }
  }
  free_posteriors(&q);
}

/* Step 9, reduction weights: none / sum -> 1, mean_batch -> 1/B,
 * mean -> 1/(B max(U_b,1)), mean_volume -> 1/max(sum_b U_b, 1). */
static void reduction_weights(int64_t B, const int64_t* Ulen, int reduction, double* wts) {
  int64_t sumU = 0;
  for (int64_t b = 0; b < B; ++b) sumU += Ulen[b];
  for (int64_t b = 0; b < B; ++b) {
    double wb = 1.0;
    if (reduction == RED_MEAN_BATCH) wb = 1.0 / (double)B;
    if (reduction == RED_MEAN) wb = 1.0 / ((double)B * (double)(Ulen[b] > 1 ? Ulen[b] : 1));
    if (reduction == RED_MEAN_VOLUME) wb = 1.0 / (double)(sumU > 1 ? sumU : 1);
    wts[b] = wb;
  }
}

static void utt_alloc(utt_t* w, int64_t T, int64_t U, int64_t D) {
  w->T = T;
  w->U = U;
  int64_t nn = T * (U + 1);
  size_t sz = (size_t)(nn > 0 ? nn : 1);
  w->lse_h = (double*)malloc(sizeof(double) * sz);
  w->lse_g = (double*)malloc(sizeof(double) * sz);
  w->lp_blank = (double*)malloc(sizeof(double) * sz);
  w->lp_label = (double*)malloc(sizeof(double) * sz);
  w->lam = (double*)malloc(sizeof(double) * sz * (size_t)D);
  w->alpha = (double*)malloc(sizeof(double) * sz);
  w->beta = (double*)malloc(sizeof(double) * sz);
}

static void utt_free(utt_t* w) {
  free(w->lse_h);
  free(w->lse_g);
  free(w->lp_blank);
  free(w->lp_label);
  free(w->lam);
  free(w->alpha);
  free(w->beta);
}

/*
 * Run the oracle on a whole batch.
 *
 * dtype: 0 fp32, 1 fp16, 2 bf16 (raw storage of the logits), 3 fp64 (for finite-difference pins).
 * tok / dur: token logits [B,Tmax,U1max,V] and duration logits [B,Tmax,U1max,D], element
 *   strides ts* / ds* for the first three dimensions, unit stride in the last one.
 * labels: [B, >= U1max-1] int64 with row stride lab_stride (-100 padding is never read).
 * Tlen / Ulen: [B] int64.  durations: [D] distinct non-negative ints, at least one > 0.
 * reduction: 0 none, 1 sum, 2 mean, 3 mean_batch, 4 mean_volume.
 *
 * Outputs (any may be NULL):
 *   loss_utt[B]   -log P per utterance (NaN for a data error, +inf if no path exists)
 *   loss_red[1]   reduced loss (for 'none' the sum of loss_utt)
 *   logp_a[B], logp_b[B]  log P from the alpha terminal and from beta(0,0)
 *   status[B]     data-error / infeasible bits
 *   weight[B]     per-utterance gradient weight w_b of the reduction
 *   node outputs  see node_out_t
 *   gtok [B,Tmax,U1max,V], gdur [B,Tmax,U1max,D]  contiguous float64 gradient of the
 *                 reduced loss ('none': of the sum of per-utterance losses); zeros at
 *                 padded nodes.
 *   rows[nrows] + rtok[nrows][V] + rdur[nrows][D]  gradient rows at selected node
 *                 indices (b*Tmax + t)*U1max + u only (zeros at padded nodes).
 * threads: OpenMP threads (<= 0: library default).  Returns 0.
 */
int tdt_oracle_run(int dtype, int64_t B, int64_t Tmax, int64_t U1max, int64_t V, int64_t D, const void* tok,
                   int64_t ts0, int64_t ts1, int64_t ts2, const void* dur, int64_t ds0, int64_t ds1, int64_t ds2,
                   const int64_t* labels, int64_t lab_stride, const int64_t* Tlen, const int64_t* Ulen,
                   const int32_t* durations, int32_t blank, double sigma, int reduction, double* loss_utt,
                   double* loss_red, double* logp_a, double* logp_b, int32_t* status, double* weight,
                   double* n_lse_h, double* n_lse_g, double* n_alpha, double* n_beta, double* n_occ,
                   double* n_cblank, double* n_clabel, double* n_cdur, double* gtok, double* gdur,
                   const int64_t* rows, int64_t nrows, double* rtok, double* rdur, int threads) {
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
  problem_t p = {dtype, B,   Tmax, U1max,      V,    D,    tok,        ts0,   ts1, ts2,
                 dur,   ds0, ds1,  ds2,        labels, lab_stride, Tlen, Ulen, durations, blank, sigma};
  node_out_t no = {n_lse_h, n_lse_g, n_alpha, n_beta, n_occ, n_cblank, n_clabel, n_cdur};
  const int64_t N = B * Tmax * U1max;
  if (gtok) memset(gtok, 0, sizeof(double) * (size_t)(N * V));
  if (gdur) memset(gdur, 0, sizeof(double) * (size_t)(N * D));
  if (rtok) memset(rtok, 0, sizeof(double) * (size_t)(nrows * V));
  if (rdur) memset(rdur, 0, sizeof(double) * (size_t)(nrows * D));
  if (n_alpha)
    for (int64_t n = 0; n < N; ++n) n_alpha[n] = -INFINITY;
  if (n_beta)
    for (int64_t n = 0; n < N; ++n) n_beta[n] = -INFINITY;
  double* per = (double*)malloc(sizeof(double) * (size_t)(B > 0 ? B : 1));
  int* st = (int*)calloc((size_t)(B > 0 ? B : 1), sizeof(int));
  double* wts = (double*)malloc(sizeof(double) * (size_t)(B > 0 ? B : 1));
  reduction_weights(B, Ulen, reduction, wts);

  for (int64_t b = 0; b < B; ++b) {
    st[b] = utterance_status(&p, b);
    if (logp_a) logp_a[b] = NAN;
    if (logp_b) logp_b[b] = NAN;
    if (st[b]) {
      per[b] = NAN;
      continue;
    }
    utt_t w;
    utt_alloc(&w, Tlen[b], Ulen[b], D);
    int64_t nn = w.T * (w.U + 1);
    node_log_probs(&p, b, &w);
    forward_alpha(&p, &w);
    backward_beta(&p, &w);
    if (logp_a) logp_a[b] = w.logp_alpha;
    if (logp_b) logp_b[b] = w.logp_beta;
    double logP = w.logp_beta;
    /* Step 6: loss_b = -log P.  No path (log P = -inf) gives +inf and zero gradients. */
    per[b] = -logP;
    if (logP == -INFINITY) {
      st[b] |= ST_INFEASIBLE;
      /* keep alpha/beta for inspection, no gradients */
      if (n_alpha || n_beta || n_lse_h || n_lse_g) {
        for (int64_t idx = 0; idx < nn; ++idx) {
          int64_t t = idx / (w.U + 1), u = idx % (w.U + 1);
          int64_t n = node_index(&p, b, t, u);
          if (n_alpha) n_alpha[n] = w.alpha[idx];
          if (n_beta) n_beta[n] = w.beta[idx];
          if (n_lse_h) n_lse_h[n] = w.lse_h[idx];
          if (n_lse_g) n_lse_g[n] = w.lse_g[idx];
        }
      }
    } else {
      node_posteriors_and_grads(&p, b, &w, logP, wts[b], &no, gtok, gdur, rows, nrows, rtok, rdur);
    }
    utt_free(&w);
  }

  double red = 0.0;
  for (int64_t b = 0; b < B; ++b) red += (reduction == RED_NONE ? 1.0 : wts[b]) * per[b];
  if (loss_red) loss_red[0] = red;
  for (int64_t b = 0; b < B; ++b) {
    if (loss_utt) loss_utt[b] = per[b];
    if (status) status[b] = st[b];
    if (weight) weight[b] = wts[b];
  }
  free(per);
  free(st);
  free(wts);
  return 0;
}

/*
 * Session form of the same computation, for batches whose full float64 gradient does not
 * fit in host memory: tdt_oracle_open runs steps 1-7 and 9 for every utterance and keeps
 * their per-node results; tdt_oracle_rows then writes the gradient rows (step 8) of a
 * range of padded node indices (b*Tmax + t)*U1max + u, zeros at padded nodes and for
 * utterances with a data error or no alignment, exactly as tdt_oracle_run writes them.
 * The logits, labels, lengths and durations passed to tdt_oracle_open must stay alive and
 * unchanged until tdt_oracle_close.
 */
typedef struct {
  problem_t p;
  int64_t B;
  int* st;
  double* wts;
  double* per;
  utt_t* w;    /* [B]; only for utterances with st == 0 and a finite log P */
  post_t* q;   /* [B] */
  int* live;   /* [B]: 1 when w[b] and q[b] hold results */
} session_t;

void* tdt_oracle_open(int dtype, int64_t B, int64_t Tmax, int64_t U1max, int64_t V, int64_t D, const void* tok,
                      int64_t ts0, int64_t ts1, int64_t ts2, const void* dur, int64_t ds0, int64_t ds1, int64_t ds2,
                      const int64_t* labels, int64_t lab_stride, const int64_t* Tlen, const int64_t* Ulen,
                      const int32_t* durations, int32_t blank, double sigma, int reduction, double* loss_utt,
                      double* loss_red, int32_t* status, int threads) {
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
  session_t* s = (session_t*)calloc(1, sizeof(session_t));
  problem_t p = {dtype, B,   Tmax, U1max,      V,    D,    tok,        ts0,   ts1, ts2,
                 dur,   ds0, ds1,  ds2,        labels, lab_stride, Tlen, Ulen, durations, blank, sigma};
  s->p = p;
  s->B = B;
  size_t nb = (size_t)(B > 0 ? B : 1);
  s->st = (int*)calloc(nb, sizeof(int));
  s->wts = (double*)malloc(sizeof(double) * nb);
  s->per = (double*)malloc(sizeof(double) * nb);
  s->w = (utt_t*)calloc(nb, sizeof(utt_t));
  s->q = (post_t*)calloc(nb, sizeof(post_t));
  s->live = (int*)calloc(nb, sizeof(int));
  reduction_weights(B, Ulen, reduction, s->wts);
  for (int64_t b = 0; b < B; ++b) {
    s->st[b] = utterance_status(&s->p, b);
    if (s->st[b]) {
      s->per[b] = NAN;
      continue;
    }
    utt_t* w = &s->w[b];
    utt_alloc(w, Tlen[b], Ulen[b], D);
    node_log_probs(&s->p, b, w);
    forward_alpha(&s->p, w);
    backward_beta(&s->p, w);
    double logP = w->logp_beta;
    s->per[b] = -logP;
    if (logP == -INFINITY) {
      s->st[b] |= ST_INFEASIBLE;
      utt_free(w);
      continue;
    }
    s->q[b] = node_posteriors(&s->p, w, logP);
    s->live[b] = 1;
  }
  double red = 0.0;
  for (int64_t b = 0; b < B; ++b) red += (reduction == RED_NONE ? 1.0 : s->wts[b]) * s->per[b];
  if (loss_red) loss_red[0] = red;
  for (int64_t b = 0; b < B; ++b) {
    if (loss_utt) loss_utt[b] = s->per[b];
    if (status) status[b] = s->st[b];
  }
  return s;
}

/* Gradient rows of the padded node indices [first, first + count) into rtok [count][V]
 * and rdur [count][D] (either may be NULL).  Returns 0, or -1 for a range outside the batch. */
int tdt_oracle_rows(void* handle, int64_t first, int64_t count, double* rtok, double* rdur) {
  session_t* s = (session_t*)handle;
  const problem_t* p = &s->p;
  const int64_t per_b = p->Tmax * p->U1max;
  if (first < 0 || count < 0 || first + count > s->B * per_b) return -1;
  if (rtok) memset(rtok, 0, sizeof(double) * (size_t)(count * p->V));
  if (rdur) memset(rdur, 0, sizeof(double) * (size_t)(count * p->D));
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t j = 0; j < count; ++j) {
    int64_t n = first + j;
    int64_t b = n / per_b;
    if (!s->live[b]) continue;
    int64_t t = (n / p->U1max) % p->Tmax;
    int64_t u = n % p->U1max;
    if (t >= s->w[b].T || u > s->w[b].U) continue;
    gradient_row(p, b, &s->w[b], &s->q[b], t, u, s->wts[b], rtok ? rtok + j * p->V : NULL,
                 rdur ? rdur + j * p->D : NULL);
  }
  return 0;
}

void tdt_oracle_close(void* handle) {
  session_t* s = (session_t*)handle;
  if (!s) return;
  for (int64_t b = 0; b < s->B; ++b) {
    if (s->live[b]) {
      utt_free(&s->w[b]);
      free_posteriors(&s->q[b]);
    }
  }
  free(s->st);
  free(s->wts);
  free(s->per);
  free(s->w);
  free(s->q);
  free(s->live);
  free(s);
}

/* Number of OpenMP threads a parallel region of this library uses. */
int tdt_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
