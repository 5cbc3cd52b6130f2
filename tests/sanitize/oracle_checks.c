/*
 * Drives the oracle's C (oracle/kda_oracle.c) for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer: small forwards over ragged and empty packed sequences,
 * head and column selections, decode steps, the backward and the DPLR forward, and
 * the argument rejections. Checks that T decode steps reproduce a T-token forward
 * and that every output is finite. Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_forward_ex(const float *q, const float *k, const float *v, const float *log_alpha, const float *beta,
                          const double *initial_state, const int64_t *seq_starts, int num_seqs, int H, int dk, int dv,
                          const int *heads, int n_heads_sel, int col_begin, int col_end, double *o_sel,
                          double *final_sel, int num_threads, int flags, double qk_eps);
int kda_oracle_decode_step_ex(const float *q, const float *k, const float *v, const float *log_alpha,
                              const float *beta, double *state, double *o, int N, int H, int dk, int dv,
                              int num_threads, int flags, double qk_eps);
int kda_oracle_backward(const float *q, const float *k, const float *v, const float *log_alpha, const float *beta,
                        const double *initial_state, const int64_t *seq_starts, int num_seqs, int H, int dk, int dv,
                        const float *d_o, const double *d_final, double *dq, double *dk_out, double *dv_out,
                        double *dlog_alpha, double *dbeta, double *d_initial, int num_threads);
int dplr_oracle_forward(const float *q, const float *k, const float *v, const float *a, const float *b,
                        const float *log_alpha, const double *initial_state, const int64_t *seq_starts, int num_seqs,
                        int H, int dk, int dv, const int *heads, int n_heads_sel, int col_begin, int col_end,
                        double *o_sel, double *final_sel, int num_threads);

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static float urand(void) { /* xorshift64*, uniform in [-1, 1) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (float)((double)((rng * 0x2545f4914f6cdd1dull) >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}
static float *frand(size_t n, float scale, float shift) {
  float *p = malloc(n * sizeof *p);
  for (size_t i = 0; i < n; ++i) p[i] = scale * urand() + shift;
  return p;
}
static int finite_all(const double *p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

int main(void) {
  enum { H = 3, DK = 8, DV = 6, T = 41, NS = 4 };
  int failures = 0;
  const int64_t starts[NS + 1] = {0, 0, 17, 18, T}; /* an empty, a 17-, a 1- and a 23-token sequence */
  float *q = frand((size_t)T * H * DK, 0.3f, 0.f), *k = frand((size_t)T * H * DK, 0.3f, 0.f);
  float *v = frand((size_t)T * H * DV, 1.f, 0.f), *la = frand((size_t)T * H * DK, 0.2f, -0.3f);
  float *beta = frand((size_t)T * H, 0.4f, 0.5f), *a = frand((size_t)T * H * DK, 0.2f, 0.f);
  float *b = frand((size_t)T * H * DK, 0.2f, 0.f), *d_o = frand((size_t)T * H * DV, 1.f, 0.f);
  double *s0 = malloc(sizeof(double) * NS * H * DK * DV), *d_fin = malloc(sizeof(double) * NS * H * DK * DV);
  for (int i = 0; i < NS * H * DK * DV; ++i) {
    s0[i] = 0.1 * urand();
    d_fin[i] = urand();
  }
  double *o = calloc((size_t)T * H * DV, sizeof(double)), *fin = calloc((size_t)NS * H * DK * DV, sizeof(double));
  if (kda_oracle_forward_ex(q, k, v, la, beta, s0, starts, NS, H, DK, DV, NULL, 0, 0, DV, o, fin, 2, 0, 0.0) != 0 ||
      !finite_all(o, (size_t)T * H * DV) || !finite_all(fin, (size_t)NS * H * DK * DV)) {
    printf("FAIL forward\n");
    ++failures;
  }
  /* one head, columns 2..5, every prologue flag */
  const int heads[1] = {2};
  double *o1 = calloc((size_t)T * DV, sizeof(double)), *f1 = calloc((size_t)NS * DK * DV, sizeof(double));
  if (kda_oracle_forward_ex(q, k, v, la, beta, s0, starts, NS, H, DK, DV, heads, 1, 2, 5, o1, f1, 1, 7, 1e-6) != 0) {
    printf("FAIL forward selection\n");
    ++failures;
  }
  /* decode: the last sequence token by token reproduces its forward outputs */
  const int n = 3, t0 = (int)starts[n], len = (int)(starts[n + 1] - starts[n]);
  double *st = malloc(sizeof(double) * H * DK * DV), *od = malloc(sizeof(double) * H * DV);
  memcpy(st, s0 + (size_t)n * H * DK * DV, sizeof(double) * H * DK * DV);
  double worst = 0.0;
  for (int t = 0; t < len; ++t) {
    const size_t tk = (size_t)(t0 + t);
    if (kda_oracle_decode_step_ex(q + tk * H * DK, k + tk * H * DK, v + tk * H * DV, la + tk * H * DK,
                                  beta + tk * H, st, od, 1, H, DK, DV, 1, 0, 0.0) != 0) {
      printf("FAIL decode\n");
      ++failures;
      break;
    }
    for (int i = 0; i < H * DV; ++i) worst = fmax(worst, fabs(od[i] - o[tk * H * DV + i]));
  }
  for (int i = 0; i < H * DK * DV; ++i) worst = fmax(worst, fabs(st[i] - fin[(size_t)n * H * DK * DV + i]));
  if (!(worst < 1e-12)) {
    printf("FAIL decode against forward: %g\n", worst);
    ++failures;
  }
  /* backward and DPLR */
  double *g[6];
  const size_t gn[6] = {(size_t)T * H * DK, (size_t)T * H * DK, (size_t)T * H * DV, (size_t)T * H * DK,
                        (size_t)T * H, (size_t)NS * H * DK * DV};
  for (int i = 0; i < 6; ++i) g[i] = calloc(gn[i], sizeof(double));
  if (kda_oracle_backward(q, k, v, la, beta, s0, starts, NS, H, DK, DV, d_o, d_fin, g[0], g[1], g[2], g[3], g[4],
                          g[5], 2) != 0) {
    printf("FAIL backward\n");
    ++failures;
  }
  for (int i = 0; i < 6; ++i)
    if (!finite_all(g[i], gn[i])) {
      printf("FAIL backward gradient %d not finite\n", i);
      ++failures;
    }
  if (dplr_oracle_forward(q, k, v, a, b, la, s0, starts, NS, H, DK, DV, NULL, 0, 0, DV, o, fin, 2) != 0 ||
      !finite_all(o, (size_t)T * H * DV)) {
    printf("FAIL dplr\n");
    ++failures;
  }
  /* rejections */
  const int64_t bad[3] = {0, 5, 3};
  if (kda_oracle_forward_ex(q, k, v, la, beta, NULL, bad, 2, H, DK, DV, NULL, 0, 0, DV, o, fin, 1, 0, 0.0) != -1 ||
      kda_oracle_forward_ex(q, k, v, la, beta, NULL, starts, NS, H, DK, DV, NULL, 0, 4, 2, o, fin, 1, 0, 0.0) != -1 ||
      kda_oracle_decode_step_ex(NULL, k, v, la, beta, st, od, 1, H, DK, DV, 1, 0, 0.0) != -1) {
    printf("FAIL rejections\n");
    ++failures;
  }
  free(q), free(k), free(v), free(la), free(beta), free(a), free(b), free(d_o), free(s0), free(d_fin);
  free(o), free(fin), free(o1), free(f1), free(st), free(od);
  for (int i = 0; i < 6; ++i) free(g[i]);
  printf("%d failures\n", failures);
  return failures != 0;
}
