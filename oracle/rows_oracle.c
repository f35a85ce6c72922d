/* Row-softmax oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain double-precision CPU statements of the row primitives on a
 * materialised (rows x cols) score matrix. Only the tests, the smoke check and
 * the benchmark's CPU baseline use them; the library never links or calls
 * them, and they share no code with the HIP path.
 *
 * What they compute, per row i (row-major float input x[i][j], j < cols):
 *
 *   admitted(j)   all j                                  softmax_rows, logsumexp_rows
 *                 mask[i][j] != 0                        masked softmax
 *                 j <= r + cols - rows_per_matrix        scaled causal softmax, r = i mod rows
 *                 (bottom-right causal, as in attention)
 *   s_j  = x_j           (unscaled ops)
 *        = scale * x_j   (scaled op; an input of -infinity stays -infinity)
 *   m    = max over admitted j of s_j
 *   l    = sum over admitted j of exp(s_j - m)           (j ascending)
 *   p_j  = exp(s_j - m) / l for admitted j, 0 otherwise
 *   lse  = m + log(l)                                    (natural log)
 *
 * Sources: pulsatrix HIPBackend page, `softmax_rows` (max-subtracted row
 * softmax) and `logsumexp_rows` (per-row log-sum-exp, max-subtracted);
 * TorchLean "CUDA Buffer Kernels FFI" page, stable row-wise hard-masked
 * softmax (max and denominator over admitted entries only, blocked entries
 * exactly zero, a row with nothing admitted all zeros); MicroGPT
 * CuBLASBackend page, `fused_attn_softmax` (scale, causal mask and softmax in
 * one pass).
 *
 * A row whose admitted scores are all -infinity, or that admits nothing
 * (including cols = 0), has p = 0 everywhere and lse = -infinity, the log of
 * an empty sum. Admitted inputs are finite or -infinity; blocked inputs may be
 * anything (NaN included) and never reach the arithmetic.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>

/* Planted mistakes for the pin tests (ROWS_PLANT_*); normal builds define none. */

static int causal_admits(long r, long j, long rows, long cols) {
#if defined(ROWS_PLANT_TOP_LEFT)
  return j <= r;
#else
  return j <= r + cols - rows;
#endif
}

/* One row. admit_kind: 0 all, 1 mask, 2 causal (r, rows given). p and lse may be NULL. */
static void oracle_softmax_row(const float* x, const float* mask, int admit_kind, long r, long rows,
                               long cols, int scaled, double scale, double* p, double* lse) {
  double m = -INFINITY;
  for (long j = 0; j < cols; ++j) {
    int ok = admit_kind == 0 ? 1 : admit_kind == 1 ? (mask[j] != 0.0f) : causal_admits(r, j, rows, cols);
#if defined(ROWS_PLANT_MASK_IN_MAX)
    ok = 1;
#endif
    if (!ok) continue;
    double s = (double)x[j];
    if (scaled && !(s == -INFINITY)) s *= scale;
    if (s > m) m = s;
  }
  if (m == -INFINITY) {
    if (p)
      for (long j = 0; j < cols; ++j) p[j] = 0.0;
#if defined(ROWS_PLANT_EMPTY_UNIFORM)
    if (p && cols > 0)
      for (long j = 0; j < cols; ++j) p[j] = 1.0 / (double)cols;
#endif
    if (lse) *lse = -INFINITY;
    return;
  }
#if defined(ROWS_PLANT_NO_MAX)
  m = 0.0;
#endif
  double l = 0.0;
  for (long j = 0; j < cols; ++j) {
    const int ok = admit_kind == 0 ? 1 : admit_kind == 1 ? (mask[j] != 0.0f) : causal_admits(r, j, rows, cols);
    double e = 0.0;
    if (ok) {
      double s = (double)x[j];
      if (scaled && !(s == -INFINITY)) s *= scale;
      e = exp(s - m);
    }
    if (p) p[j] = e;
    l += e;
  }
  if (p)
    for (long j = 0; j < cols; ++j) p[j] /= l;
  if (lse) {
#if defined(ROWS_PLANT_LSE_LOG2)
    *lse = (m + log(l)) / log(2.0);
#else
    *lse = m + log(l);
#endif
  }
}

int oracle_softmax_rows(const float* in, long rows, long cols, double* out) {
  if (rows < 0 || cols < 0) return -1;
#pragma omp parallel for schedule(dynamic, 16)
  for (long i = 0; i < rows; ++i)
    oracle_softmax_row(in + (size_t)i * cols, 0, 0, 0, 0, cols, 0, 1.0, out + (size_t)i * cols, 0);
  return 0;
}

int oracle_logsumexp_rows(const float* in, long rows, long cols, double* out) {
  if (rows < 0 || cols < 0) return -1;
#pragma omp parallel for schedule(dynamic, 16)
  for (long i = 0; i < rows; ++i)
    oracle_softmax_row(in + (size_t)i * cols, 0, 0, 0, 0, cols, 0, 1.0, 0, out + i);
  return 0;
}

int oracle_masked_softmax_rows(const float* in, const float* mask, long rows, long cols, double* out) {
  if (rows < 0 || cols < 0) return -1;
#pragma omp parallel for schedule(dynamic, 16)
  for (long i = 0; i < rows; ++i)
    oracle_softmax_row(in + (size_t)i * cols, mask + (size_t)i * cols, 1, 0, 0, cols, 0, 1.0,
                       out + (size_t)i * cols, 0);
  return 0;
}

/* batch matrices of rows x cols each; causal = 0 admits every entry. */
int oracle_scaled_causal_softmax(const float* in, long batch, long rows, long cols, double scale,
                                 int causal, double* out) {
  if (batch < 0 || rows < 0 || cols < 0) return -1;
  const long n = batch * rows;
#pragma omp parallel for schedule(dynamic, 16)
  for (long i = 0; i < n; ++i)
    oracle_softmax_row(in + (size_t)i * cols, 0, causal ? 2 : 0, i % (rows > 0 ? rows : 1), rows,
                       cols, 1, scale, out + (size_t)i * cols, 0);
  return 0;
}

/* Softmax backward from its output (pulsatrix HIPBackend `softmax_rows_backward`;
 * scaled, MicroGPT `fused_attn_softmax_backward`): for each row,
 *   dot = sum_k y[k] * dy[k],   dx[j] = scale * y[j] * (dy[j] - dot),
 * in double, k ascending. scale = 1 is the plain softmax backward; for the fused
 * scale + mask + softmax forward it is the forward's scale (masked entries have
 * y = 0 and so get 0). */
int oracle_softmax_rows_backward(const float* y, const float* dy, long rows, long cols,
                                 double scale, double* dx) {
  if (rows < 0 || cols < 0) return -1;
#pragma omp parallel for schedule(static)
  for (long r = 0; r < rows; ++r) {
    const float* yr = y + (size_t)r * cols;
    const float* gr = dy + (size_t)r * cols;
    double* o = dx + (size_t)r * cols;
    double dot = 0.0;
    for (long k = 0; k < cols; ++k) dot += (double)yr[k] * (double)gr[k];
#if defined(ROWS_PLANT_BWD_NO_DOT)
    dot = 0.0;
#endif
    for (long j = 0; j < cols; ++j) {
#if defined(ROWS_PLANT_BWD_SIGN)
      o[j] = scale * (double)yr[j] * (dot - (double)gr[j]);
#else
      o[j] = scale * (double)yr[j] * ((double)gr[j] - dot);
#endif
    }
  }
  return 0;
}
