/*
 * CPU oracle in plain C for the Skip-Softmax (BLASST) FlashAttention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, constant or helper with the HIP
 * library.
 *
 * Two parts, both written from the method's description:
 *   oracle_dense_head     softmax attention of one head in double precision,
 *                         the definition written out.
 *   oracle_skip_head_f32  the tiled skip-softmax recurrence in single
 *                         precision ("Skip-Softmax" design document of
 *                         vLLM-Omni, section "Algorithm"; "Skip-Softmax" page
 *                         of the vLLM-Omni documentation, sections "The
 *                         online-softmax pass" and "The skip test").
 *   oracle_skip_mask_f32  the same recurrence reduced to what the tile
 *                         decisions depend on (scores, tile maxima, the vote
 *                         and the running maximum of the kept tiles).
 *
 * Readings taken where the pages leave a step open (the same ones the
 * Python oracle takes): the running maximum is the one held before the tile
 * is absorbed; the test is strict; a block of query rows skips a tile only
 * when every valid row passes; skipped tiles change nothing, m included;
 * tiles are visited in ascending key order; ln(lambda) is given already
 * rounded to float.
 *
 * Single precision, step by step: a score is the float sum over channels of
 * q * k, in channel order, times the scale (one rounding each); the margin
 * is float(tile_max - m); exponentials are expf; l and O are float sums.
 * Inputs are float copies of bf16 values, which float holds exactly.
 *
 * Plain loops, no intrinsics; OpenMP over query blocks (rows are
 * independent).  Planted mistakes for the tests are compiled in with
 * -DORACLE_MUTANT=n (see tests/test_c_oracle.py); the default build has none.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

/* Threads a parallel region of this library uses (1 without OpenMP). */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Softmax attention of one head, every row: o = softmax(scale q k^T) v and
 * lse = log sum exp(scale q k^T), natural log.  q, k: [S][D]; v: [S][Dv];
 * o: [S][Dv]; lse: [S].  Returns 0, or -1 when scratch memory is missing. */
int oracle_dense_head(const double* q, const double* k, const double* v, int S, int D, int Dv, double scale,
                      double* o, double* lse) {
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    if (s == NULL) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int i = 0; i < S; ++i) {
        double mx = -INFINITY;
        for (int j = 0; j < S; ++j) {
          double dot = 0.0;
#if ORACLE_MUTANT == 8
          for (int t = 0; t < D; ++t) dot += k[(size_t)i * D + t] * q[(size_t)j * D + t];   /* q and k swapped */
#else
          for (int t = 0; t < D; ++t) dot += q[(size_t)i * D + t] * k[(size_t)j * D + t];
#endif
          s[j] = scale * dot;
          if (s[j] > mx) mx = s[j];
        }
        double den = 0.0;
        double* oi = o + (size_t)i * Dv;
        for (int t = 0; t < Dv; ++t) oi[t] = 0.0;
        for (int j = 0; j < S; ++j) {
          const double p = exp(s[j] - mx);
          den += p;
          for (int t = 0; t < Dv; ++t) oi[t] += p * v[(size_t)j * Dv + t];
        }
        for (int t = 0; t < Dv; ++t) oi[t] /= den;
        lse[i] = mx + log(den);
      }
      free(s);
    }
  }
  return failed ? -1 : 0;
}

/* The streaming pass of one head with the per-tile skip test.
 *
 * q, k: [S][D], v: [S][Dv] (float).  vote = 0 disables the test (lambda = 0);
 * otherwise a tile is skipped for a block when every valid row i of the
 * block has float(tile_max_i - m_i) < ln_lambda.  qblocks[nb]: the blocks of
 * block_q rows to compute.  forced (nullable, [nb][nkt], 1 = skip) replaces
 * the decisions.  Outputs, per computed block: o [nb][block_q][Dv] = O / l,
 * lse [nb][block_q] = m + ln l (padding rows included, their values
 * meaningless), skipped [nb][nkt], margin [nb][nkt] = max over valid rows of
 * tile_max - m (+inf on a block's first tile).  Returns 0, or -1 when scratch
 * memory is missing. */
static int skip_head_f32(const float* q, const float* k, const float* v, int S, int D, int Dv, float scale, int vote,
                         float ln_lambda, int block_q, int block_k, const int64_t* qblocks, int nb,
                         const uint8_t* forced, int mask_only, float* o, float* lse, uint8_t* skipped,
                         float* margin) {
  const int nkt = (S + block_k - 1) / block_k;
  int failed = 0;
#pragma omp parallel
  {
    float* s = (float*)malloc(sizeof(float) * (size_t)block_q * block_k);
    float* m = (float*)malloc(sizeof(float) * (size_t)block_q);
    float* l = (float*)malloc(sizeof(float) * (size_t)block_q);
    float* tmax = (float*)malloc(sizeof(float) * (size_t)block_q);
    if (s == NULL || m == NULL || l == NULL || tmax == NULL) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int b = 0; b < nb; ++b) {
        const int r0 = (int)qblocks[b] * block_q;
        float* ob = mask_only ? NULL : o + (size_t)b * block_q * Dv;
        for (int i = 0; i < block_q; ++i) {
          m[i] = -INFINITY;
          l[i] = 0.f;
        }
        if (!mask_only) memset(ob, 0, sizeof(float) * (size_t)block_q * Dv);
        for (int kt = 0; kt < nkt; ++kt) {
          const int c0 = kt * block_k;
          const int c1 = (c0 + block_k < S) ? c0 + block_k : S;
          const int nc = c1 - c0;
          /* 1. scores of the tile, always; 2. each row's tile maximum */
          for (int i = 0; i < block_q; ++i) {
            const int row = r0 + i;
            float mx = -INFINITY;
            for (int c = 0; c < nc; ++c) {
              float dot = 0.f;
              if (row < S)
                for (int t = 0; t < D; ++t) dot += q[(size_t)row * D + t] * k[(size_t)(c0 + c) * D + t];
#if ORACLE_MUTANT == 4
              const float sc = dot;   /* scale dropped */
#else
              const float sc = dot * scale;
#endif
              s[i * block_k + c] = sc;
              if (sc > mx) mx = sc;
            }
            tmax[i] = mx;
          }
          /* 3. the vote: every valid row's margin below ln(lambda), strictly */
          float worst = -INFINITY;
          for (int i = 0; i < block_q; ++i) {
#if ORACLE_MUTANT == 5
            const int votes = 1;   /* padding rows vote */
#else
            const int votes = r0 + i < S;
#endif
            if (!votes) continue;
#if ORACLE_MUTANT == 2
            const float mref = tmax[i] > m[i] ? tmax[i] : m[i];   /* maximum taken after absorbing the tile */
#else
            const float mref = m[i];
#endif
            const float d = (mref == -INFINITY) ? INFINITY : tmax[i] - mref;
            if (d > worst) worst = d;
          }
          margin[(size_t)b * nkt + kt] = worst;
          int skip;
          if (forced != NULL)
            skip = forced[(size_t)b * nkt + kt] != 0;
          else if (!vote)
            skip = 0;
          else
#if ORACLE_MUTANT == 1
            skip = worst <= ln_lambda;   /* non-strict test */
#else
            skip = worst < ln_lambda;
#endif
          skipped[(size_t)b * nkt + kt] = (uint8_t)skip;
          if (skip) {
#if ORACLE_MUTANT == 6
            for (int i = 0; i < block_q; ++i)
              if (tmax[i] > m[i]) m[i] = tmax[i];   /* skipped tiles still raise m */
#endif
            continue;   /* 4. a skipped tile leaves m, l and O untouched */
          }
          /* 5. a kept tile is absorbed exactly (only its maximum when just the
           * decisions are wanted: l and O never feed back into them) */
          for (int i = 0; i < block_q; ++i) {
            const float mn = tmax[i] > m[i] ? tmax[i] : m[i];
            if (mask_only) {
              m[i] = mn;
              continue;
            }
#if ORACLE_MUTANT == 3
            const float alpha = 1.f;   /* l and O not rescaled */
#else
            const float alpha = expf(m[i] - mn);   /* 0 on the first kept tile */
#endif
            float rs = 0.f;
            float* oi = ob + (size_t)i * Dv;
            for (int t = 0; t < Dv; ++t) oi[t] *= alpha;
            for (int c = 0; c < nc; ++c) {
              const float p = expf(s[i * block_k + c] - mn);
              rs += p;
              for (int t = 0; t < Dv; ++t) oi[t] += p * v[(size_t)(c0 + c) * Dv + t];
            }
            l[i] = alpha * l[i] + rs;
            m[i] = mn;
          }
        }
        for (int i = 0; i < block_q && !mask_only; ++i) {
          float* oi = ob + (size_t)i * Dv;
          for (int t = 0; t < Dv; ++t) oi[t] /= l[i];
#if ORACLE_MUTANT == 7
          lse[(size_t)b * block_q + i] = logf(l[i]);   /* the running maximum left out */
#else
          lse[(size_t)b * block_q + i] = m[i] + logf(l[i]);
#endif
        }
      }
    }
    free(s);
    free(m);
    free(l);
    free(tmax);
  }
  return failed ? -1 : 0;
}

int oracle_skip_head_f32(const float* q, const float* k, const float* v, int S, int D, int Dv, float scale, int vote,
                         float ln_lambda, int block_q, int block_k, const int64_t* qblocks, int nb,
                         const uint8_t* forced, float* o, float* lse, uint8_t* skipped, float* margin) {
  return skip_head_f32(q, k, v, S, D, Dv, scale, vote, ln_lambda, block_q, block_k, qblocks, nb, forced, 0, o, lse,
                       skipped, margin);
}

/* The same recurrence for the tile decisions and margins alone: the scores,
 * each row's tile maximum, the vote, and for a kept tile the running maximum
 * m' = max(m, tile_max).  The decisions depend on nothing else (l and O never
 * enter the test), so they equal oracle_skip_head_f32's, at about half the
 * work (no exponentials, no P.V).  v, o and lse are not used. */
int oracle_skip_mask_f32(const float* q, const float* k, int S, int D, float scale, int vote, float ln_lambda,
                         int block_q, int block_k, const int64_t* qblocks, int nb, uint8_t* skipped, float* margin) {
  return skip_head_f32(q, k, NULL, S, D, 0, scale, vote, ln_lambda, block_q, block_k, qblocks, nb, NULL, 1, NULL, NULL,
                       skipped, margin);
}
