/*
 * Driver for the sanitizer build of the fp64 oracle (oracle/sdpa_f64.c),
 * compiled with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_oracle_sanitize.py and run on the CPU.  It exercises every
 * entry point over tiny and ragged shapes, both masks, all rows and row
 * subsets (first and last rows included), one thread and more threads than
 * rows, and the argument errors; it checks what any correct result has
 * (finite outputs, probability rows summing to one, masked probabilities
 * exactly zero, the error codes).  Memory and undefined-behaviour errors are
 * the sanitizers' to report.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int kbo_sdpa_rows(const float *Q, const float *K, const float *V, int64_t BH, int64_t S, int64_t d,
                  int causal, double scale, const int64_t *rows, int64_t nrows, double *O, int nthreads);
int kbo_probs_rows(const float *Q, const float *K, const float *V, int64_t BH, int64_t S, int64_t d,
                   int causal, double scale, const int64_t *rows, int64_t nrows, double *P, int nthreads);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static float draw(void) { /* uniform in [-2, 2), exact in fp32 */
  state = state * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((int32_t)(state >> 40) - (1 << 23)) / (float)(1 << 22);
}

static int failures = 0;
#define CHECK(c, ...)                      \
  do {                                     \
    if (!(c)) {                            \
      fprintf(stderr, __VA_ARGS__);        \
      fputc('\n', stderr);                 \
      ++failures;                          \
    }                                      \
  } while (0)

static void one_shape(int64_t BH, int64_t S, int64_t d) {
  const int64_t n = BH * S * d;
  /* exact-size heap buffers, so any overrun is an ASan report */
  float *Q = malloc(n * sizeof(float)), *K = malloc(n * sizeof(float)), *V = malloc(n * sizeof(float));
  for (int64_t i = 0; i < n; ++i) {
    Q[i] = draw();
    K[i] = draw();
    V[i] = draw();
  }
  const int64_t nall = BH * S;
  int64_t sub[3] = {nall - 1, 0, nall / 2};
  for (int causal = 0; causal <= 1; ++causal) {
    for (int variant = 0; variant < 2; ++variant) {
      const int64_t *rows = variant ? sub : NULL;
      const int64_t nr = variant ? 3 : nall;
      for (int nt = 1; nt <= 9; nt += 4) {
        double *O = malloc(nr * d * sizeof(double));
        double *P = malloc(nr * S * sizeof(double));
        int rc = kbo_sdpa_rows(Q, K, V, BH, S, d, causal, 0.0, rows, nr, O, nt);
        CHECK(rc == 0, "sdpa rc %d (BH %ld S %ld d %ld)", rc, (long)BH, (long)S, (long)d);
        rc = kbo_probs_rows(Q, K, V, BH, S, d, causal, 0.0, rows, nr, P, nt);
        CHECK(rc == 0, "probs rc %d", rc);
        for (int64_t r = 0; r < nr; ++r) {
          const int64_t i = (rows ? rows[r] : r) % S;
          double sum = 0.0;
          for (int64_t j = 0; j < S; ++j) {
            const double p = P[r * S + j];
            CHECK(p >= 0.0 && p <= 1.0, "probability out of range");
            if (causal && j > i) CHECK(p == 0.0, "masked probability %g at i %ld j %ld", p, (long)i, (long)j);
            sum += p;
          }
          CHECK(fabs(sum - 1.0) <= 1e-12, "row sum %.17g", sum);
          for (int64_t k = 0; k < d; ++k) CHECK(isfinite(O[r * d + k]), "non-finite output");
        }
        free(O);
        free(P);
      }
    }
  }
  /* argument errors: nothing is computed or written */
  int64_t bad[2] = {0, nall};
  double out[1];
  CHECK(kbo_sdpa_rows(Q, K, V, BH, S, d, 0, 0.0, bad, 2, out, 2) == -3, "row out of range accepted");
  bad[1] = -1;
  CHECK(kbo_sdpa_rows(Q, K, V, BH, S, d, 0, 0.0, bad, 2, out, 2) == -3, "negative row accepted");
  CHECK(kbo_sdpa_rows(Q, K, V, 0, S, d, 0, 0.0, NULL, 0, out, 1) == -2, "BH = 0 accepted");
  CHECK(kbo_sdpa_rows(NULL, K, V, BH, S, d, 0, 0.0, NULL, 0, out, 1) == -2, "NULL Q accepted");
  CHECK(kbo_probs_rows(Q, K, V, BH, S, d, 0, 0.0, NULL, 0, NULL, 1) == -2, "NULL output accepted");
  free(Q);
  free(K);
  free(V);
}

int main(void) {
  const int64_t shapes[][3] = {{1, 1, 1}, {1, 2, 1}, {2, 3, 2}, {3, 17, 5}, {2, 64, 32}, {1, 129, 64}};
  for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) one_shape(shapes[s][0], shapes[s][1], shapes[s][2]);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle sanitizer driver: all checks passed\n");
  return 0;
}
