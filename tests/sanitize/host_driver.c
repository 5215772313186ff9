/* CPU driver for the library's host code (validation, sizing, workspace
 * carving) under AddressSanitizer and UndefinedBehaviorSanitizer: kvc_plan
 * on valid and invalid problems, and every prefill entry point with
 * arguments that are rejected before anything is launched, so no GPU is
 * needed.  Exit status 0 when every call returned the expected status. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvc.h"

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                                    \
    }                                                              \
  } while (0)

static kvc_problem prob(int n_seq, const int64_t *starts, const double *ret, int NL, int H, int G,
                        int d, int T) {
  kvc_problem p;
  memset(&p, 0, sizeof p);
  p.n_seq = n_seq;
  p.n_layers = NL;
  p.n_kv_heads = H;
  p.gqa_group = G;
  p.head_dim = d;
  p.n_window_q = 32;
  p.dtype = KVC_BF16;
  p.seq_start = starts;
  p.retention = ret;
  p.k_stride[0] = p.v_stride[0] = (int64_t)H * T * d;
  p.k_stride[1] = p.v_stride[1] = (int64_t)T * d;
  p.k_stride[2] = p.v_stride[2] = d;
  return p;
}

int main(void) {
  kvc_params prm = {0.5, 0.7, 32, 0.5, KVC_POOL_SEQUENCE, KVC_SCORE_MEAN};
  int64_t rows = 0;
  size_t ws = 0;
  const int lens[] = {100, 1000, 4096, 16385, 32768, 49999, 65535, 65536};
  for (size_t i = 0; i < sizeof lens / sizeof lens[0]; ++i) {
    const int64_t st[2] = {0, lens[i]};
    const double r[1] = {0.9};
    kvc_problem p = prob(1, st, r, 48, 4, 8, 128, lens[i]);
    CHECK(kvc_plan(&p, &prm, &rows, &ws) == KVC_OK);
    CHECK(rows > 0 && ws > 0);
  }
  /* ragged batch of 64 sequences, and the rejections */
  int64_t st64[65];
  double r64[64];
  for (int i = 0; i <= 64; ++i) st64[i] = (int64_t)i * 1000;
  for (int i = 0; i < 64; ++i) r64[i] = 0.2 + 0.01 * i;
  kvc_problem p = prob(64, st64, r64, 2, 2, 4, 64, 64000);
  CHECK(kvc_plan(&p, &prm, &rows, &ws) == KVC_OK);
  p.n_seq = 65;
  CHECK(kvc_plan(&p, &prm, &rows, &ws) != KVC_OK);
  const int64_t st1[2] = {0, 65537};
  const double r1[1] = {0.5};
  p = prob(1, st1, r1, 2, 2, 4, 64, 65537);
  CHECK(kvc_plan(&p, &prm, NULL, NULL) == KVC_ERR_UNSUPPORTED);
  p.seq_start = NULL;
  CHECK(kvc_plan(&p, &prm, NULL, NULL) == KVC_ERR_INVALID_ARG);
  CHECK(kvc_plan(NULL, &prm, NULL, NULL) == KVC_ERR_INVALID_ARG);
  const int64_t st2[2] = {0, 4096};
  p = prob(1, st2, r1, 2, 2, 4, 64, 4096);
  kvc_params bad = prm;
  bad.alpha = 2.0;
  CHECK(kvc_plan(&p, &bad, NULL, NULL) == KVC_ERR_INVALID_ARG);
  /* entry points refused before any launch */
  void *fake = (void *)(uintptr_t)(1 << 20);
  CHECK(kvc_compress(&p, &prm, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, 0,
                     NULL) == KVC_ERR_WORKSPACE);
  CHECK(kvc_compress(&p, &prm, NULL, fake, fake, fake, fake, fake, fake, fake, fake, fake, 1 << 30,
                     NULL) == KVC_ERR_INVALID_ARG);
  CHECK(kvc_compress_layers(&p, &prm, 1, 1, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                            fake, 1 << 30, NULL) == KVC_ERR_INVALID_ARG);
  CHECK(kvc_scores(&p, &prm, fake, fake, fake, fake, 0, NULL) == KVC_ERR_WORKSPACE);
  CHECK(kvc_smooth(&p, &prm, NULL, fake, fake, NULL, 0, NULL) == KVC_ERR_INVALID_ARG);
  CHECK(kvc_select(&p, &prm, fake, NULL, fake, fake, NULL) == KVC_ERR_INVALID_ARG);
  CHECK(kvc_gather(&p, &prm, fake, fake, fake, fake, NULL, fake, NULL) == KVC_ERR_INVALID_ARG);
  /* two 65536-token sequences: a workspace beyond the static array */
  const int64_t st3[3] = {0, 65536, 131072};
  const double r3[2] = {0.2, 0.2};
  kvc_problem big = prob(2, st3, r3, 48, 4, 8, 128, 131072);
  CHECK(kvc_compress_noalloc(&big, &prm, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                             NULL) == KVC_ERR_WORKSPACE);
  for (int s = 0; s < 8; ++s) CHECK(kvc_status_str((kvc_status)s) != NULL);
  CHECK(kvc_last_hip_error() == 0);
  puts("host driver ok");
  return 0;
}
