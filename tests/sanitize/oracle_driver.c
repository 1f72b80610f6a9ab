/* Driver for the sanitizer build of the plain-C oracle (tests only): runs
 * every exported function on small inputs, ragged shapes included, and
 * checks a few results, so that AddressSanitizer and UndefinedBehavior-
 * Sanitizer see every code path (dense, recurrence with and without the
 * vote, forced mask, decisions-only mode).  Exit status 0 = all checks
 * passed; the sanitizers abort on the first error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_threads(void);
int oracle_dense_head(const double* q, const double* k, const double* v, int S, int D, int Dv, double scale,
                      double* o, double* lse);
int oracle_skip_head_f32(const float* q, const float* k, const float* v, int S, int D, int Dv, float scale, int vote,
                         float ln_lambda, int block_q, int block_k, const int64_t* qblocks, int nb,
                         const uint8_t* forced, float* o, float* lse, uint8_t* skipped, float* margin);
int oracle_skip_mask_f32(const float* q, const float* k, int S, int D, float scale, int vote, float ln_lambda,
                         int block_q, int block_k, const int64_t* qblocks, int nb, uint8_t* skipped, float* margin);

static unsigned rng_state = 12345u;
static float urand(void) {
  rng_state = rng_state * 1664525u + 1013904223u;
  return (float)((rng_state >> 8) & 0xFFFF) / 65536.0f - 0.5f;
}

int main(void) {
  const int shapes[][4] = {{1, 8, 8, 4}, {37, 8, 5, 7}, {300, 16, 64, 128}, {129, 16, 64, 128}};
  int failures = 0;
  for (unsigned c = 0; c < sizeof(shapes) / sizeof(shapes[0]); ++c) {
    const int S = shapes[c][0], D = shapes[c][1], bq = shapes[c][2], bk = shapes[c][3];
    const int nqb = (S + bq - 1) / bq, nkt = (S + bk - 1) / bk;
    float* q = malloc(sizeof(float) * S * D);
    float* k = malloc(sizeof(float) * S * D);
    float* v = malloc(sizeof(float) * S * D);
    double *qd = malloc(sizeof(double) * S * D), *kd = malloc(sizeof(double) * S * D), *vd = malloc(sizeof(double) * S * D);
    for (int i = 0; i < S * D; ++i) {
      q[i] = 4.f * urand();
      k[i] = 4.f * urand();
      v[i] = urand();
      qd[i] = q[i];
      kd[i] = k[i];
      vd[i] = v[i];
    }
    double* od = malloc(sizeof(double) * S * D);
    double* lsed = malloc(sizeof(double) * S);
    if (oracle_dense_head(qd, kd, vd, S, D, D, 0.3, od, lsed) != 0) ++failures;
    int64_t* qb = malloc(sizeof(int64_t) * nqb);
    for (int i = 0; i < nqb; ++i) qb[i] = i;
    float* o = malloc(sizeof(float) * nqb * bq * D);
    float* lse = malloc(sizeof(float) * nqb * bq);
    uint8_t* sk = malloc((size_t)nqb * nkt);
    uint8_t* sk2 = malloc((size_t)nqb * nkt);
    float* mg = malloc(sizeof(float) * nqb * nkt);
    float* mg2 = malloc(sizeof(float) * nqb * nkt);
    const float lns[] = {-4.f, -1.f, 2.f};
    for (int li = 0; li < 3; ++li) {
      if (oracle_skip_head_f32(q, k, v, S, D, D, 0.3f, 1, lns[li], bq, bk, qb, nqb, NULL, o, lse, sk, mg) != 0) ++failures;
      if (oracle_skip_mask_f32(q, k, S, D, 0.3f, 1, lns[li], bq, bk, qb, nqb, sk2, mg2) != 0) ++failures;
      for (int i = 0; i < nqb * nkt; ++i)
        if (sk[i] != sk2[i] || !(mg[i] == mg2[i] || (isinf(mg[i]) && isinf(mg2[i])))) ++failures;
      if (oracle_skip_head_f32(q, k, v, S, D, D, 0.3f, 0, 0.f, bq, bk, qb, nqb, sk, o, lse, sk2, mg2) != 0) ++failures;
    }
    /* no vote: the recurrence is dense attention */
    if (oracle_skip_head_f32(q, k, v, S, D, D, 0.3f, 0, 0.f, bq, bk, qb, nqb, NULL, o, lse, sk, mg) != 0) ++failures;
    for (int r = 0; r < S; ++r)
      if (fabs((double)lse[r] - lsed[r]) > 1e-3) ++failures;
    free(q); free(k); free(v); free(qd); free(kd); free(vd); free(od); free(lsed);
    free(qb); free(o); free(lse); free(sk); free(sk2); free(mg); free(mg2);
  }
  printf("oracle driver: %d threads, %d failures\n", oracle_threads(), failures);
  return failures == 0 ? 0 : 1;
}
