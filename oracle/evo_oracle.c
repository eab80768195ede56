/*
 * evo_oracle.c -- plain, slow, fp64 CPU oracle for 3D (triangle / MSA-row)
 * attention with an additively broadcast pair bias.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (MegaFold, gist.science technical summary, Methodik section 1
 * "EvoFlash-3D": exact attention over the 2D pair representation, with a pair
 * bias added by broadcast to every row; the memory-efficient kernel must give
 * the same numbers as this direct form).  For every attention row r, head h,
 * query j and key k, in the kernel frame:
 *
 *   S[r,h,j,k] = (sum_c q[r,j,h,c] k[r,k,h,c]) / sqrt(d) + bias[h,j,k] + mask[r,k]
 *   P[r,h,j,:] = softmax_k S[r,h,j,:]
 *   O[r,j,h,c] = sum_k P[r,h,j,k] v[r,k,h,c]
 *   lse[r,h,j] = log sum_k exp S[r,h,j,k]                      (natural log)
 *
 * and, for the loss L = sum O * dO (mask receives no gradient):
 *
 *   dV[r,k,h,c]  = sum_j P[j,k] dO[r,j,h,c]
 *   dP[j,k]      = sum_c dO[r,j,h,c] v[r,k,h,c]
 *   D[j]         = sum_k P[j,k] dP[j,k]
 *   dS[j,k]      = P[j,k] (dP[j,k] - D[j])
 *   dQ[r,j,h,c]  = sum_k dS[j,k] k[r,k,h,c] / sqrt(d)
 *   dK[r,k,h,c]  = sum_j dS[j,k] q[r,j,h,c] / sqrt(d)
 *   dBias[h,j,k] = sum_r dS[r,h,j,k]        (summed in increasing r)
 *
 * The softmax is the textbook one: the full row of logits is formed, its
 * maximum subtracted, exponentiated and divided by the sum.  No online
 * softmax, no tiling.  Each (r, h) logit slab [N, N] is materialised in full.
 *
 * Readings where the pages are silent (all are listed in the design notes):
 *  - a row whose keys are all masked (every logit -inf) has O = 0, lse = -inf
 *    and contributes nothing to any gradient;
 *  - transpose = 1 changes only the addressing of q, k, v, O, dO, dQ, dK, dV:
 *    element (r, p, h, c) lives at physical [p, r, h, c]; bias, mask and lse
 *    stay in the kernel frame;
 *  - bias and mask may be NULL (treated as 0).
 *
 * Row subsets: `rows` (sorted, strictly increasing) restricts the work to those
 * attention rows; outputs of other rows are left untouched and dBias sums only
 * the listed rows.  NULL means all rows.
 *
 * Parallelism: OpenMP over (h, j) or (h, k) inside one row; rows are visited in
 * increasing order, so every sum has a fixed order and the results do not
 * depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static inline int64_t phys(int64_t R, int64_t N, int64_t H, int64_t D, int transpose,
                           int64_t r, int64_t p, int64_t h) {
  int64_t pos = transpose ? (p * R + r) : (r * N + p);
  return (pos * H + h) * D;
}

int evo_oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* One softmax row (r, h, j): fills srow[N] with P[j,:] and returns lse.
 * Returns -INFINITY (and P = 0) when every logit is -inf. */
static double softmax_row(int64_t R, int64_t N, int64_t H, int64_t D, int transpose,
                          const double* q, const double* k, const double* bias,
                          const double* mask, int64_t r, int64_t h, int64_t j,
                          double* srow) {
  const double scale = 1.0 / sqrt((double)D);
  const double* qj = q + phys(R, N, H, D, transpose, r, j, h);
  double m = -INFINITY;
  for (int64_t kk = 0; kk < N; ++kk) {
    const double* kv = k + phys(R, N, H, D, transpose, r, kk, h);
    double dot = 0.0;
    for (int64_t c = 0; c < D; ++c) dot += qj[c] * kv[c];
    double s = dot * scale;
    if (bias) s += bias[(h * N + j) * N + kk];
    if (mask) s += mask[r * N + kk];
    srow[kk] = s;
    if (s > m) m = s;
  }
  if (m == -INFINITY) {
    for (int64_t kk = 0; kk < N; ++kk) srow[kk] = 0.0;
    return -INFINITY;
  }
  double z = 0.0;
  for (int64_t kk = 0; kk < N; ++kk) {
    srow[kk] = exp(srow[kk] - m);
    z += srow[kk];
  }
  for (int64_t kk = 0; kk < N; ++kk) srow[kk] /= z;
  return m + log(z);
}

/* Forward for one attention row r: P slab [H][N][N], O and lse. */
static void forward_row(int64_t R, int64_t N, int64_t H, int64_t D, int transpose,
                        const double* q, const double* k, const double* v,
                        const double* bias, const double* mask, int64_t r,
                        double* pslab, double* o, double* lse) {
#pragma omp parallel for schedule(static)
  for (int64_t hj = 0; hj < H * N; ++hj) {
    const int64_t h = hj / N, j = hj % N;
    double* prow = pslab + (h * N + j) * N;
    const double l = softmax_row(R, N, H, D, transpose, q, k, bias, mask, r, h, j, prow);
    if (lse) lse[(r * H + h) * N + j] = l;
    if (o) {
      double* oj = o + phys(R, N, H, D, transpose, r, j, h);
      for (int64_t c = 0; c < D; ++c) oj[c] = 0.0;
      for (int64_t kk = 0; kk < N; ++kk) {
        const double p = prow[kk];
        const double* vk = v + phys(R, N, H, D, transpose, r, kk, h);
        for (int64_t c = 0; c < D; ++c) oj[c] += p * vk[c];
      }
    }
  }
}

int evo_oracle_fwd(int64_t R, int64_t N, int64_t H, int64_t D, int transpose,
                   const double* q, const double* k, const double* v,
                   const double* bias, const double* mask,
                   const int64_t* rows, int64_t nrows,
                   double* o, double* lse) {
  if (R <= 0 || N <= 0 || H <= 0 || D <= 0 || !q || !k || !v) return 1;
  double* pslab = (double*)malloc(sizeof(double) * (size_t)(H * N * N));
  if (!pslab) return 2;
  const int64_t count = rows ? nrows : R;
  for (int64_t t = 0; t < count; ++t) {
    const int64_t r = rows ? rows[t] : t;
    forward_row(R, N, H, D, transpose, q, k, v, bias, mask, r, pslab, o, lse);
  }
  free(pslab);
  return 0;
}

int evo_oracle_bwd(int64_t R, int64_t N, int64_t H, int64_t D, int transpose,
                   const double* q, const double* k, const double* v,
                   const double* bias, const double* mask, const double* dout,
                   const int64_t* rows, int64_t nrows,
                   double* dq, double* dk, double* dv, double* dbias) {
  if (R <= 0 || N <= 0 || H <= 0 || D <= 0 || !q || !k || !v || !dout) return 1;
  const double scale = 1.0 / sqrt((double)D);
  const size_t slab = (size_t)(H * N * N);
  double* pslab = (double*)malloc(sizeof(double) * slab);
  double* dsslab = (double*)malloc(sizeof(double) * slab);
  if (!pslab || !dsslab) { free(pslab); free(dsslab); return 2; }
  if (dbias) memset(dbias, 0, sizeof(double) * slab);

  const int64_t count = rows ? nrows : R;
  for (int64_t t = 0; t < count; ++t) {
    const int64_t r = rows ? rows[t] : t;
    /* Forward: softmax rows P[h][j][:]. */
    forward_row(R, N, H, D, transpose, q, k, v, bias, mask, r, pslab, NULL, NULL);

    /* dP, D, dS and dQ, one (h, j) row at a time. */
#pragma omp parallel for schedule(static)
    for (int64_t hj = 0; hj < H * N; ++hj) {
      const int64_t h = hj / N, j = hj % N;
      const double* prow = pslab + (h * N + j) * N;
      double* dsrow = dsslab + (h * N + j) * N;
      const double* doj = dout + phys(R, N, H, D, transpose, r, j, h);
      double dsum = 0.0;
      for (int64_t kk = 0; kk < N; ++kk) {
        const double* vk = v + phys(R, N, H, D, transpose, r, kk, h);
        double dp = 0.0;
        for (int64_t c = 0; c < D; ++c) dp += doj[c] * vk[c];
        dsrow[kk] = dp;                 /* holds dP until D is known */
        dsum += prow[kk] * dp;
      }
      for (int64_t kk = 0; kk < N; ++kk) dsrow[kk] = prow[kk] * (dsrow[kk] - dsum);
      if (dq) {
        double* dqj = dq + phys(R, N, H, D, transpose, r, j, h);
        for (int64_t c = 0; c < D; ++c) dqj[c] = 0.0;
        for (int64_t kk = 0; kk < N; ++kk) {
          const double* kv = k + phys(R, N, H, D, transpose, r, kk, h);
          for (int64_t c = 0; c < D; ++c) dqj[c] += dsrow[kk] * kv[c];
        }
        for (int64_t c = 0; c < D; ++c) dqj[c] *= scale;
      }
    }

    /* dK and dV, one (h, k) column at a time, summing over queries j in order. */
#pragma omp parallel for schedule(static)
    for (int64_t hk = 0; hk < H * N; ++hk) {
      const int64_t h = hk / N, kk = hk % N;
      double* dkk = dk ? dk + phys(R, N, H, D, transpose, r, kk, h) : NULL;
      double* dvk = dv ? dv + phys(R, N, H, D, transpose, r, kk, h) : NULL;
      for (int64_t c = 0; c < D; ++c) {
        if (dkk) dkk[c] = 0.0;
        if (dvk) dvk[c] = 0.0;
      }
      for (int64_t j = 0; j < N; ++j) {
        const double p = pslab[(h * N + j) * N + kk];
        const double ds = dsslab[(h * N + j) * N + kk];
        const double* qj = q + phys(R, N, H, D, transpose, r, j, h);
        const double* doj = dout + phys(R, N, H, D, transpose, r, j, h);
        for (int64_t c = 0; c < D; ++c) {
          if (dkk) dkk[c] += ds * qj[c];
          if (dvk) dvk[c] += p * doj[c];
        }
      }
      if (dkk)
        for (int64_t c = 0; c < D; ++c) dkk[c] *= scale;
    }

    /* dBias: add this row's dS slab; rows arrive in increasing order. */
    if (dbias) {
#pragma omp parallel for schedule(static)
      for (int64_t hj = 0; hj < H * N; ++hj)
        for (int64_t kk = 0; kk < N; ++kk) dbias[hj * N + kk] += dsslab[hj * N + kk];
    }
  }
  free(pslab);
  free(dsslab);
  return 0;
}
