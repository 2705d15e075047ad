/*
 * ssd_oracle.c -- fp64 reference of the Mamba-2 SSD forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the oracle the GPU path is checked
 * against. Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load it; the product library never does, and this file
 * shares no code, header or constant with the HIP sources.
 *
 * What it computes (plain definition, token by token, in double precision):
 *
 *   for every sequence s and head h, with group g = h / (H / G):
 *     st  <- initial state of (s, h)  (P x N), or zeros
 *     for each token t of s, in order:
 *       a        = exp(dt[t,h] * A[h])
 *       st[p,n]  = a * st[p,n] + dt[t,h] * x[t,h,p] * B[t,g,n]
 *       y[t,h,p] = sum_n C[t,g,n] * st[p,n] + D[h] * x[t,h,p]
 *     final state of (s, h) <- st
 *
 * Sources, by page:
 *  - tj-hxxt.cn long read of "Mamba: Linear-Time Sequence Modeling with
 *    Selective State Spaces", part III "Selective State Space Models":
 *    sub-section (2) makes B, C and the step size input dependent (one value
 *    per token); sub-section 3 ("parameters of the selection mechanism",
 *    item on A) gives the discretised decay as exp(step * A).
 *  - the same page, part III, item 2.3 "Boundary Resetting": independent
 *    packed sequences must not leak state into one another, hence the reset to
 *    the initial state at every sequence start.
 *  - kuaisou "mamba model explained" snippets: C, B and the input play the
 *    roles of query, key and value of linear attention, so the output reads
 *    the state through C and the input enters through B.
 *  - QbitAI "Mamba-2" article (srwj168 repost), section "Mamba-2: stronger
 *    learning, faster training and inference": several heads share one
 *    multi-input SSM; B and C are shared by the heads of one group.
 * The input term dt * B * x (Euler rule, no zero-order-hold factor), the
 * scalar A per head, the contiguous head-to-group map and the skip term D
 * are readings the pages leave open; they are listed with the oracle's
 * pins in the design notes.
 *
 * Optional snapshots: with snap_every = Q > 0 the state held just before the
 * tokens at offsets 0, Q, 2Q, ... of each sequence is copied out. That is the
 * state entering each chunk of length Q, numbered sequence by sequence.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* Returns 0 on success, a negative number for a malformed call. */
int ssd_oracle_forward(int64_t nseq, const int64_t *seq_start,
                       const int64_t *seq_len, int64_t H, int64_t P, int64_t N,
                       int64_t G, const double *x, const double *dt,
                       const double *A, const double *B, const double *C,
                       const double *D, const double *h0, double *y,
                       double *h_final, int64_t snap_every, double *snaps,
                       int nthreads) {
  if (nseq < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0)
    return -1;
  if (snap_every < 0 || (snap_every > 0 && snaps == NULL)) return -2;
  for (int64_t s = 0; s < nseq; ++s)
    if (seq_len[s] < 0 || seq_start[s] < 0) return -3;

  /* First snapshot index of each sequence. */
  int64_t *snap_base = (int64_t *)calloc((size_t)nseq + 1, sizeof(int64_t));
  if (!snap_base) return -4;
  for (int64_t s = 0; s < nseq; ++s)
    snap_base[s + 1] =
        snap_base[s] + (snap_every > 0 ? ceil_div(seq_len[s], snap_every) : 0);

  const int64_t heads_per_group = H / G;
  const int64_t pairs = nseq * H;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t pair = 0; pair < pairs; ++pair) {
    const int64_t s = pair / H, h = pair % H, g = h / heads_per_group;
    double *st = (double *)malloc((size_t)(P * N) * sizeof(double));
    if (!st) {
      failed = 1;
      continue;
    }
    if (h0)
      memcpy(st, h0 + (s * H + h) * P * N, (size_t)(P * N) * sizeof(double));
    else
      memset(st, 0, (size_t)(P * N) * sizeof(double));
    const double d_skip = D ? D[h] : 0.0;

    for (int64_t i = 0; i < seq_len[s]; ++i) {
      const int64_t t = seq_start[s] + i;
      if (snap_every > 0 && i % snap_every == 0) {
        double *dst = snaps + ((snap_base[s] + i / snap_every) * H + h) * P * N;
        memcpy(dst, st, (size_t)(P * N) * sizeof(double));
      }
      const double step = dt[t * H + h];
      const double decay = exp(step * A[h]);
      const double *xt = x + (t * H + h) * P;
      const double *bt = B + (t * G + g) * N;
      const double *ct = C + (t * G + g) * N;
      double *yt = y + (t * H + h) * P;
      for (int64_t p = 0; p < P; ++p) {
        const double u = step * xt[p];
        double *row = st + p * N;
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          row[n] = decay * row[n] + u * bt[n];
          acc += ct[n] * row[n];
        }
        yt[p] = acc + d_skip * xt[p];
      }
    }
    if (h_final)
      memcpy(h_final + (s * H + h) * P * N, st, (size_t)(P * N) * sizeof(double));
    free(st);
  }
  free(snap_base);
  return failed ? -5 : 0;
}
