/* CPU driver for the oracle's C code under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every entry point on small inputs of odd and
 * even lengths, including the degenerate ones (constant rows, zero scores,
 * full retention, windows covering the row) and the rejected arguments.
 * Exit status 0 when every call returned what it should; a sanitizer
 * report aborts the process. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int kvo_scores(int gw, int L, int d, const double *q, const double *k, double *s);
int kvo_dft(int L, const double *s, double *re, double *im);
int kvo_sss(int L, const double *s, double alpha, double rho, int kstar_in, double *s_hat,
            int *kstar, double *energy, double *lp_out);
int kvo_budget(int n, const float *S, int L, double retention, double base_ratio, int w,
               int *b);
int kvo_select(int L, const double *s_hat, int w, int b, int *kept);

static unsigned long long st = 88172645463325252ull;
static double rnd(void) { /* xorshift64, uniform in [0, 1) */
  st ^= st << 13;
  st ^= st >> 7;
  st ^= st << 17;
  return (double)(st >> 11) * (1.0 / 9007199254740992.0);
}

#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                               \
    }                                                         \
  } while (0)

int main(void) {
  const int lens[] = {1, 2, 3, 7, 64, 65, 100, 127, 256};
  for (size_t li = 0; li < sizeof lens / sizeof lens[0]; ++li) {
    const int L = lens[li], d = 8, gw = 5;
    double *q = malloc(sizeof(double) * gw * d), *k = malloc(sizeof(double) * L * d);
    double *s = malloc(sizeof(double) * L), *sh = malloc(sizeof(double) * L);
    double *re = malloc(sizeof(double) * (L / 2 + 1)), *im = malloc(sizeof(double) * (L / 2 + 1));
    double *en = malloc(sizeof(double) * (L / 2 + 1)), *lp = malloc(sizeof(double) * L);
    int *kept = malloc(sizeof(int) * L);
    for (int i = 0; i < gw * d; ++i) q[i] = rnd() - 0.5;
    for (int i = 0; i < L * d; ++i) k[i] = rnd() - 0.5;
    CHECK(kvo_scores(gw, L, d, q, k, s) == 0);
    double tot = 0.0;
    for (int j = 0; j < L; ++j) tot += s[j];
    CHECK(fabs(tot - 1.0) < 1e-12);
    CHECK(kvo_dft(L, s, re, im) == 0);
    int ks = -1;
    CHECK(kvo_sss(L, s, 0.6, 0.7, -1, sh, &ks, en, lp) == 0);
    CHECK(ks >= 0 && ks <= L / 2);
    CHECK(kvo_sss(L, s, 0.6, 0.7, L / 2, sh, &ks, NULL, NULL) == 0);
    for (int j = 0; j < L; ++j) s[j] = 0.25;          /* constant row */
    CHECK(kvo_sss(L, s, 1.0, 0.7, -1, sh, &ks, NULL, NULL) == 0 && ks == 0);
    for (int w = 0; w <= L; w += (L > 8 ? L / 4 : 1))
      for (int b = w; b <= L; b += (L > 8 ? L / 5 : 1)) CHECK(kvo_select(L, s, w, b, kept) == 0);
    free(q); free(k); free(s); free(sh); free(re); free(im); free(en); free(lp); free(kept);
  }
  /* budgets: random, zero and capped scores; full retention */
  for (int n = 1; n <= 300; n += 37) {
    float *S = malloc(sizeof(float) * n);
    int *b = malloc(sizeof(int) * n);
    for (int rep = 0; rep < 3; ++rep) {
      for (int u = 0; u < n; ++u) S[u] = rep == 0 ? (float)rnd() : rep == 1 ? 0.0f : (u % 7 == 0);
      const int L = 4096;
      CHECK(kvo_budget(n, S, L, 0.4, 0.5, 32, b) == 0);
      long long sum = 0;
      for (int u = 0; u < n; ++u) sum += b[u];
      CHECK(sum == (long long)n * (long long)floor(0.4 * L));
      CHECK(kvo_budget(n, S, L, 1.0, 0.5, 32, b) == 0);
    }
    free(S); free(b);
  }
  /* rejected arguments */
  float bad[2] = {-1.0f, 0.5f};
  int bb[2];
  CHECK(kvo_budget(2, bad, 1024, 0.5, 0.5, 32, bb) != 0);
  CHECK(kvo_scores(0, 4, 4, NULL, NULL, NULL) != 0);
  CHECK(kvo_sss(0, NULL, 0.5, 0.7, -1, NULL, NULL, NULL, NULL) != 0);
  puts("oracle driver ok");
  return 0;
}
