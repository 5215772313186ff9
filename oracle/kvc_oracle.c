/*
 * kvc_oracle.c -- plain, slow, fp64 CPU oracle for audio prefill KV-cache
 * compression.  TEST INFRASTRUCTURE ONLY: it is loaded by tests/, by the
 * smoke check and by the CPU-baseline leg of bench.py, never by the product
 * path.  It shares no code, header, table or constant with the HIP library.
 *
 * Every function below is the plain definition of one step of the method,
 * written out with no blocking, fusion or reordering:
 *
 *   kvo_scores  observation-window attention importance per KV head
 *               (AudioKV article, section 1.2 "raw importance score"; the
 *               softmax(q K^T / sqrt(d)) form is the one written in the VoxZip
 *               digest, "Temporally Decayed KV Cache Eviction" equation)
 *   kvo_dft     direct O(L^2) real-input DFT, bins 0..floor(L/2)
 *   kvo_sss     Spectral Score Smoothing (AudioKV article, section 2.2):
 *               F = rfft(s), cumulative energy E(k), smallest k* with
 *               E(k*) >= rho * E(L/2), brick-wall low-pass keeping bins
 *               0..k*, inverse real DFT, blend (1-alpha) s + alpha lowpass
 *   kvo_budget  head-aware budget b = w + r + B_score * S / sum(S)
 *               (AudioKV article, section 3.1 and the section 5.1 config
 *               block), with the cap at L and largest-remainder rounding
 *   kvo_select  per-head top-k of the smoothed row plus the local window
 *
 * Conventions (readings taken where the pages are silent): all floating
 * point is IEEE fp64, sums run
 * in ascending index order, and the file is compiled with
 * -ffp-contract=off so that no multiply-add is fused.
 *
 * Return values: 0 on success, a negative number on a rejected input.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KVO_OK 0
#define KVO_EINVAL (-1)
#define KVO_EBUDGET (-2)
#define KVO_ENOMEM (-3)
#define KVO_EINTERNAL (-4)

/* ------------------------------------------------------------------------ */
/* Step 1: importance scores.                                                */
/* q: [gw][d] window queries of the KV head's whole GQA group (gw = G * W),  */
/* k: [L][d] audio keys.  s[j] = mean over the gw queries of softmax_j(l),   */
/* l[j] = (q . k_j) / sqrt(d), the softmax taken over all L audio keys.      */
/* ------------------------------------------------------------------------ */
int kvo_scores(int gw, int L, int d, const double *q, const double *k,
               double *s) {
  if (gw <= 0 || L <= 0 || d <= 0 || !q || !k || !s) return KVO_EINVAL;
  double *logit = (double *)malloc(sizeof(double) * (size_t)L);
  if (!logit) return KVO_ENOMEM;
  const double rs = sqrt((double)d);
  for (int j = 0; j < L; ++j) s[j] = 0.0;
  for (int g = 0; g < gw; ++g) {
    const double *qg = q + (size_t)g * d;
    double m = -INFINITY;
    for (int j = 0; j < L; ++j) {
      const double *kj = k + (size_t)j * d;
      double dot = 0.0;
      for (int c = 0; c < d; ++c) dot += qg[c] * kj[c];
      logit[j] = dot / rs;
      if (logit[j] > m) m = logit[j];
    }
    double z = 0.0;
    for (int j = 0; j < L; ++j) {
      logit[j] = exp(logit[j] - m);
      z += logit[j];
    }
    for (int j = 0; j < L; ++j) s[j] += logit[j] / z;
  }
  for (int j = 0; j < L; ++j) s[j] /= (double)gw;
  free(logit);
  return KVO_OK;
}

/* ------------------------------------------------------------------------ */
/* Direct real-input DFT.  F_k = sum_j s_j exp(-2 pi i j k / L), k=0..n,     */
/* n = floor(L/2).  The angle index (j*k) mod L is reduced exactly in        */
/* integers and looked up in an L-entry cos/sin table.                       */
/* ------------------------------------------------------------------------ */
static int twiddles(int L, double **c, double **sn) {
  *c = (double *)malloc(sizeof(double) * (size_t)L);
  *sn = (double *)malloc(sizeof(double) * (size_t)L);
  if (!*c || !*sn) {
    free(*c);
    free(*sn);
    return KVO_ENOMEM;
  }
  const double two_pi = 2.0 * 3.14159265358979323846;
  for (int m = 0; m < L; ++m) {
    (*c)[m] = cos(two_pi * (double)m / (double)L);
    (*sn)[m] = sin(two_pi * (double)m / (double)L);
  }
  return KVO_OK;
}

static void dft_with(int L, const double *s, const double *c,
                     const double *sn, double *re, double *im) {
  const int n = L / 2;
  for (int k = 0; k <= n; ++k) {
    double a = 0.0, b = 0.0;
    for (int j = 0; j < L; ++j) {
      const int64_t m = ((int64_t)j * (int64_t)k) % (int64_t)L;
      a += s[j] * c[m];
      b -= s[j] * sn[m];
    }
    re[k] = a;
    im[k] = b;
  }
}

int kvo_dft(int L, const double *s, double *re, double *im) {
  if (L <= 0 || !s || !re || !im) return KVO_EINVAL;
  double *c, *sn;
  if (twiddles(L, &c, &sn)) return KVO_ENOMEM;
  dft_with(L, s, c, sn, re, im);
  free(c);
  free(sn);
  return KVO_OK;
}

/* ------------------------------------------------------------------------ */
/* Step 2: Spectral Score Smoothing.                                         */
/*   E(k)  = sum_{i<=k} |F_i|^2, k = 0..n                                    */
/*   k*    = min{ k : E(k) >= rho * E(n) }   (or kstar_in when >= 0)         */
/*   lp    = inverse real DFT of F with bins k*+1..n set to zero; the        */
/*           imaginary parts of the DC bin and (L even) the Nyquist bin are  */
/*           ignored, as a real inverse transform does                       */
/*   s_hat = (1 - alpha) s + alpha lp                                        */
/* Optional outputs: energy [n+1], lp [L] (pass NULL to skip).               */
/* ------------------------------------------------------------------------ */
int kvo_sss(int L, const double *s, double alpha, double rho, int kstar_in,
            double *s_hat, int *kstar, double *energy, double *lp_out) {
  if (L <= 0 || !s || !s_hat || !kstar) return KVO_EINVAL;
  const int n = L / 2;
  if (kstar_in > n) return KVO_EINVAL;
  double *c, *sn;
  if (twiddles(L, &c, &sn)) return KVO_ENOMEM;
  double *re = (double *)malloc(sizeof(double) * (size_t)(n + 1));
  double *im = (double *)malloc(sizeof(double) * (size_t)(n + 1));
  double *E = (double *)malloc(sizeof(double) * (size_t)(n + 1));
  if (!re || !im || !E) {
    free(c); free(sn); free(re); free(im); free(E);
    return KVO_ENOMEM;
  }
  dft_with(L, s, c, sn, re, im);

  double acc = 0.0;
  for (int k = 0; k <= n; ++k) {
    acc += re[k] * re[k] + im[k] * im[k];
    E[k] = acc;
  }
  int ks = kstar_in;
  if (ks < 0) {
    const double target = rho * E[n];
    ks = n;
    for (int k = 0; k <= n; ++k) {
      if (E[k] >= target) {
        ks = k;
        break;
      }
    }
  }
  *kstar = ks;

  /* Bins 1..last_pair appear twice in the real inverse (k and L-k). */
  const int even = (L % 2 == 0);
  const int last_pair = even ? n - 1 : n;
  const int top = ks < last_pair ? ks : last_pair;
  for (int j = 0; j < L; ++j) {
    double v = re[0];
    for (int k = 1; k <= top; ++k) {
      const int64_t m = ((int64_t)j * (int64_t)k) % (int64_t)L;
      v += 2.0 * (re[k] * c[m] - im[k] * sn[m]);
    }
    if (even && ks == n && n > 0) v += (j % 2 == 0) ? re[n] : -re[n];
    const double lp = v / (double)L;
    if (lp_out) lp_out[j] = lp;
    s_hat[j] = (1.0 - alpha) * s[j] + alpha * lp;
  }
  if (energy)
    for (int k = 0; k <= n; ++k) energy[k] = E[k];
  free(c); free(sn); free(re); free(im); free(E);
  return KVO_OK;
}

/* ------------------------------------------------------------------------ */
/* Step 3: head-aware budget for one sequence.                               */
/* n heads (all layers x KV heads of the sequence, flattened l*H + h), each  */
/* with audio-head score S[u] >= 0.                                          */
/*   kbar  = floor(retention * L)            tokens kept per head on average */
/*   r     = floor(base_ratio * kbar)        uniform base share              */
/*   fixed = w + r                           window + base, every head       */
/*   R     = n*kbar - n*fixed                score-proportional pool         */
/* Each head's share of R is R*S_u/sum(S) (uniform when sum(S) == 0).  A     */
/* head's share may not exceed cap = L - fixed: shares that reach the cap    */
/* are fixed at the cap and the rest of the pool is split again among the    */
/* others (water-filling).  Shares are made integral by largest remainder:   */
/* every head gets floor(share), and the heads with the largest fractional   */
/* parts (ties: lower u) get one more until the pool is used up.             */
/* When kbar >= L every head keeps all L tokens.                             */
/* ------------------------------------------------------------------------ */
typedef struct {
  double frac;
  int u;
} kvo_rem;

static int rem_cmp(const void *a, const void *b) {
  const kvo_rem *x = (const kvo_rem *)a, *y = (const kvo_rem *)b;
  if (x->frac > y->frac) return -1;
  if (x->frac < y->frac) return 1;
  return (x->u > y->u) - (x->u < y->u);
}

int kvo_budget(int n, const float *S, int L, double retention,
               double base_ratio, int w, int *b) {
  if (n <= 0 || !S || !b || L <= 0 || w < 0) return KVO_EINVAL;
  if (!(retention > 0.0 && retention <= 1.0)) return KVO_EINVAL;
  if (!(base_ratio >= 0.0 && base_ratio <= 1.0)) return KVO_EINVAL;
  for (int u = 0; u < n; ++u)
    if (!(S[u] >= 0.0f) || isinf(S[u])) return KVO_EINVAL;

  const int64_t kbar = (int64_t)floor(retention * (double)L);
  if (kbar >= L) {
    for (int u = 0; u < n; ++u) b[u] = L;
    return KVO_OK;
  }
  const int64_t r = (int64_t)floor(base_ratio * (double)kbar);
  const int64_t fixed = (int64_t)w + r;
  if (L <= w || fixed > kbar) return KVO_EBUDGET;

  int64_t R = (int64_t)n * kbar - (int64_t)n * fixed;
  const int64_t cap = (int64_t)L - fixed;
  char *active = (char *)malloc((size_t)n);
  double *q = (double *)malloc(sizeof(double) * (size_t)n);
  int64_t *extra = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
  kvo_rem *rem = (kvo_rem *)malloc(sizeof(kvo_rem) * (size_t)n);
  if (!active || !q || !extra || !rem) {
    free(active); free(q); free(extra); free(rem);
    return KVO_ENOMEM;
  }
  for (int u = 0; u < n; ++u) {
    active[u] = 1;
    extra[u] = 0;
  }

  for (;;) {
    double sumA = 0.0;
    int nA = 0;
    for (int u = 0; u < n; ++u)
      if (active[u]) {
        sumA += (double)S[u];
        ++nA;
      }
    if (nA == 0) break;
    for (int u = 0; u < n; ++u) {
      if (!active[u]) continue;
      if (sumA > 0.0)
        q[u] = ((double)R * (double)S[u]) / sumA;
      else
        q[u] = (double)R / (double)nA;
    }
    int capped = 0;
    for (int u = 0; u < n; ++u)
      if (active[u] && q[u] >= (double)cap) {
        active[u] = 0;
        extra[u] = cap;
        ++capped;
      }
    if (!capped) break;
    R -= cap * (int64_t)capped;
  }

  int nA = 0;
  int64_t floors = 0;
  for (int u = 0; u < n; ++u) {
    if (!active[u]) continue;
    const double f = floor(q[u]);
    extra[u] = (int64_t)f;
    floors += extra[u];
    rem[nA].frac = q[u] - f;
    rem[nA].u = u;
    ++nA;
  }
  const int64_t deficit = R - floors;
  if (deficit < 0 || deficit > nA) {
    free(active); free(q); free(extra); free(rem);
    return KVO_EINTERNAL;
  }
  qsort(rem, (size_t)nA, sizeof(kvo_rem), rem_cmp);
  for (int64_t i = 0; i < deficit; ++i) extra[rem[i].u] += 1;

  for (int u = 0; u < n; ++u) b[u] = (int)(fixed + extra[u]);
  free(active); free(q); free(extra); free(rem);
  return KVO_OK;
}

/* ------------------------------------------------------------------------ */
/* Step 4: per-head selection.  Candidates are positions [0, L-w); the       */
/* b-w of them with the largest s_hat are kept (equal values: the lower      */
/* position first; -0.0 equals +0.0).  The last w positions are always       */
/* kept.  kept[0..b) lists the positions in ascending order.                 */
/* ------------------------------------------------------------------------ */
typedef struct {
  double v;
  int j;
} kvo_cand;

static int sel_cmp(const void *a, const void *b) {
  const kvo_cand *x = (const kvo_cand *)a, *y = (const kvo_cand *)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->j > y->j) - (x->j < y->j);
}

static int int_cmp(const void *a, const void *b) {
  const int i = *(const int *)a, j = *(const int *)b;
  return (i > j) - (i < j);
}

int kvo_select(int L, const double *s_hat, int w, int b, int *kept) {
  if (L <= 0 || !s_hat || !kept || w < 0 || w > L || b < w || b > L)
    return KVO_EINVAL;
  for (int j = 0; j < L; ++j)
    if (isnan(s_hat[j]) || isinf(s_hat[j])) return KVO_EINVAL;
  const int ncand = L - w;
  const int k = b - w;
  kvo_cand *cand =
      (kvo_cand *)malloc(sizeof(kvo_cand) * (size_t)(ncand > 0 ? ncand : 1));
  if (!cand) return KVO_ENOMEM;
  for (int j = 0; j < ncand; ++j) {
    cand[j].v = s_hat[j];
    cand[j].j = j;
  }
  qsort(cand, (size_t)ncand, sizeof(kvo_cand), sel_cmp);
  for (int t = 0; t < k; ++t) kept[t] = cand[t].j;
  qsort(kept, (size_t)k, sizeof(int), int_cmp);
  for (int t = 0; t < w; ++t) kept[k + t] = ncand + t;
  free(cand);
  return KVO_OK;
}
