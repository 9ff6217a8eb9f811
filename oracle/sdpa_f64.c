/*
 * Scaled dot-product attention, forward pass: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker that the GPU kernels
 * are compared against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; no product code path calls it.
 * It shares no code, header or constant with the GPU library.
 *
 * What it computes (kbench page, "The three GPU kernels"): for every
 * flattened batch*head slice and every query row i,
 *
 *     O[i, :] = softmax_j( scale * <Q[i,:], K[j,:]> ) . V[j, :]
 *
 * with scale = 1/sqrt(d) and the [head, seq, dim] row-major layout the page
 * states.  "causal" (kbench page, MCU request fields) is read as: key j is
 * visible to query i iff j <= i (0-based), masked keys get weight exactly 0.
 *
 * The three steps are written out separately, in the order the definition
 * gives them (scores, softmax, weighted sum of value rows).  Everything is
 * evaluated in double with libm exp; the inputs arrive as float32 values
 * (every fp32 and bf16 input is exactly representable there) and are upcast.
 * No tiling, no online rescaling, no reordering beyond the definition.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Number of keys query row i may attend to. */
static int64_t visible_count(int64_t i, int64_t S, int causal) {
    return causal ? i + 1 : S;
}

/* Step 1: s_j = scale * sum_k q[k] * K[j, k] for the visible keys j. */
static void row_scores(const float *q, const float *Kh, int64_t nvis, int64_t d,
                       double scale, double *s) {
    for (int64_t j = 0; j < nvis; ++j) {
        double dot = 0.0;
        for (int64_t k = 0; k < d; ++k)
            dot += (double)q[k] * (double)Kh[j * d + k];
        s[j] = scale * dot;
    }
}

/* Step 2: softmax over the visible scores, in place.
 * w_j = exp(s_j - m) with m = max_j s_j (subtracting m changes nothing in
 * exact arithmetic and keeps exp finite); returns Z = sum_j w_j. */
static double row_softmax_weights(double *s, int64_t nvis) {
    double m = s[0];
    for (int64_t j = 1; j < nvis; ++j)
        if (s[j] > m) m = s[j];
    double Z = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        s[j] = exp(s[j] - m);
        Z += s[j];
    }
    return Z;
}

/* Step 3: o = (sum_j w_j * V[j, :]) / Z. */
static void row_weighted_values(const double *w, double Z, const float *Vh,
                                int64_t nvis, int64_t d, double *o) {
    for (int64_t k = 0; k < d; ++k) o[k] = 0.0;
    for (int64_t j = 0; j < nvis; ++j)
        for (int64_t k = 0; k < d; ++k)
            o[k] += w[j] * (double)Vh[j * d + k];
    for (int64_t k = 0; k < d; ++k) o[k] /= Z;
}

typedef struct {
    const float *Q, *K, *V;
    int64_t BH, S, d;
    int causal;
    double scale;
    const int64_t *rows; /* flat row ids bh*S + i, or NULL for all rows */
    int64_t nrows;
    double *O; /* nrows x d output rows */
    double *P; /* nrows x S probabilities, or NULL */
    int tid, nthreads;
    int status;
} job_t;

static void *worker(void *arg) {
    job_t *jb = (job_t *)arg;
    double *s = (double *)malloc((size_t)jb->S * sizeof(double));
    double *o = (double *)malloc((size_t)jb->d * sizeof(double));
    if (!s || !o) {
        jb->status = -1;
        free(s);
        free(o);
        return NULL;
    }
    for (int64_t r = jb->tid; r < jb->nrows; r += jb->nthreads) {
        int64_t flat = jb->rows ? jb->rows[r] : r;
        int64_t bh = flat / jb->S, i = flat % jb->S;
        const float *q = jb->Q + (bh * jb->S + i) * jb->d;
        const float *Kh = jb->K + bh * jb->S * jb->d;
        const float *Vh = jb->V + bh * jb->S * jb->d;
        int64_t nvis = visible_count(i, jb->S, jb->causal);

        row_scores(q, Kh, nvis, jb->d, jb->scale, s);
        double Z = row_softmax_weights(s, nvis);
        if (jb->O) {
            row_weighted_values(s, Z, Vh, nvis, jb->d, o);
            memcpy(jb->O + r * jb->d, o, (size_t)jb->d * sizeof(double));
        }
        if (jb->P) {
            double *prow = jb->P + r * jb->S;
            for (int64_t j = 0; j < jb->S; ++j) prow[j] = j < nvis ? s[j] / Z : 0.0;
        }
    }
    free(s);
    free(o);
    return NULL;
}

static int run(const float *Q, const float *K, const float *V, int64_t BH, int64_t S,
               int64_t d, int causal, double scale, const int64_t *rows, int64_t nrows,
               double *O, double *P, int nthreads) {
    if (!Q || !K || !V || BH < 1 || S < 1 || d < 1 || (!O && !P)) return -2;
    if (!rows) nrows = BH * S;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= BH * S) return -3;
    if (scale == 0.0) scale = 1.0 / sqrt((double)d);
    if (nthreads < 1) nthreads = 1;
    if ((int64_t)nthreads > nrows) nthreads = (int)nrows;

    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    for (int t = 0; t < nthreads; ++t) {
        job_t jb = {Q, K, V, BH, S, d, causal, scale, rows, nrows, O, P, t, nthreads, 0};
        jobs[t] = jb;
    }
    int started = 0, status = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, worker, &jobs[t]) != 0) {
            status = -4;
            break;
        }
        started = t;
    }
    if (status == 0) worker(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    for (int t = 0; t < nthreads && status == 0; ++t)
        if (jobs[t].status != 0) status = jobs[t].status;
    free(jobs);
    free(th);
    return status;
}

/* O rows of SDPA in fp64.
 * Q, K, V: [BH, S, d] float32, row-major.  rows: flat ids bh*S+i to compute
 * (NULL = all BH*S rows in order); O receives nrows x d doubles in the order
 * of `rows`.  scale 0 means 1/sqrt(d).  Returns 0 on success, <0 on bad
 * arguments or allocation failure. */
int kbo_sdpa_rows(const float *Q, const float *K, const float *V, int64_t BH, int64_t S,
                  int64_t d, int causal, double scale, const int64_t *rows, int64_t nrows,
                  double *O, int nthreads) {
    return run(Q, K, V, BH, S, d, causal, scale, rows, nrows, O, NULL, nthreads);
}

/* The softmax probabilities P[i, j] of the same rows (masked keys = 0),
 * nrows x S doubles. */
int kbo_probs_rows(const float *Q, const float *K, const float *V, int64_t BH, int64_t S,
                   int64_t d, int causal, double scale, const int64_t *rows, int64_t nrows,
                   double *P, int nthreads) {
    return run(Q, K, V, BH, S, d, causal, scale, rows, nrows, NULL, P, nthreads);
}
