/* Attention-forward oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, double-precision CPU statement of what the attention forward
 * pass computes. Only the tests, the smoke check and the benchmark's CPU
 * baseline use it; the library never links or calls it, and it shares no code
 * with the HIP path.
 *
 * What it computes, per (batch b, head h) and query row i
 * (oxicuda ComputeBackend page, documentation of `attention`; the scale is read
 * as a multiplier of QK^T, whose usual value is 1/sqrt(head_dim)):
 *
 *   keys allowed to row i:  j < hi(i), hi(i) = seq_kv                       (no mask)
 *                                      hi(i) = clamp(i + seq_kv - seq_q + 1, 0, seq_kv)
 *                                                                (causal, bottom-right)
 *   s_j    = scale * sum_c q[i][c] * k[j][c]           (j < hi(i), c ascending)
 *   m      = max_j s_j                                 (max-subtracted: pulsatrix
 *                                                       softmax_rows / logsumexp_rows)
 *   l      = sum_j exp(s_j - m)                        (j ascending)
 *   o[i][c]= sum_j exp(s_j - m) * v[j][c] / l
 *   lse[i] = m + log(l)                                (natural log)
 *
 * A row with no allowed key (hi(i) = 0) is all zeros, as the TorchLean
 * hard-masked softmax defines it, and its log-sum-exp is the log of an empty
 * sum, -infinity.
 *
 * Inputs are float32 arrays holding the exact input values (bfloat16 inputs
 * widen to float32 exactly); all arithmetic is in double. Layout: contiguous
 * row-major q, o [B][H][seq_q][D]; k, v [B][H][seq_kv][D]; lse [B][H][seq_q].
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared oracle/attention_oracle.c -o oracle/liboracle.so -lm
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>

/* Planted mistakes: the pin tests compile this file with one ORACLE_PLANT_*
 * macro defined and check that some pin fails. Normal builds define none. */

/* Number of keys query row i may attend. */
static long allowed_keys(long i, long seq_q, long seq_kv, int causal) {
  if (!causal) return seq_kv;
#if defined(ORACLE_PLANT_STRICT_MASK)
  long hi = i + (seq_kv - seq_q);
#elif defined(ORACLE_PLANT_TOP_LEFT)
  long hi = i + 1;
#else
  long hi = i + (seq_kv - seq_q) + 1;
#endif
  if (hi < 0) hi = 0;
  if (hi > seq_kv) hi = seq_kv;
  return hi;
}

/* One query row, straight from the definition. s is scratch of length >= hi. */
static void oracle_row(const float* q_row, const float* k_bh, const float* v_bh, long hi, long d,
                       long seq_kv, double scale, double* s, double* o_row, double* lse) {
#if defined(ORACLE_PLANT_SWAP_KV)
  const float* t = k_bh; k_bh = v_bh; v_bh = t;
#endif
  (void)seq_kv;
  if (hi == 0) {
    for (long c = 0; c < d; ++c) o_row[c] = 0.0;
#if defined(ORACLE_PLANT_EMPTY_LSE_ZERO)
    *lse = 0.0;
#else
    *lse = -INFINITY;
#endif
    return;
  }
  for (long j = 0; j < hi; ++j) {
    double dot = 0.0;
#if defined(ORACLE_PLANT_TRANSPOSED_K)
    for (long c = 0; c < d; ++c) dot += (double)q_row[c] * (double)k_bh[c * seq_kv + j];
#else
    for (long c = 0; c < d; ++c) dot += (double)q_row[c] * (double)k_bh[j * d + c];
#endif
#if defined(ORACLE_PLANT_DROP_SCALE)
    s[j] = dot;
#elif defined(ORACLE_PLANT_DIVIDE_SCALE)
    s[j] = dot / scale;
#else
    s[j] = scale * dot;
#endif
  }
  double m = s[0];
  for (long j = 1; j < hi; ++j)
    if (s[j] > m) m = s[j];
#if defined(ORACLE_PLANT_NO_MAX)
  m = 0.0;
#endif
  double l = 0.0;
  for (long j = 0; j < hi; ++j) {
    s[j] = exp(s[j] - m);
    l += s[j];
  }
  for (long c = 0; c < d; ++c) {
    double acc = 0.0;
    for (long j = 0; j < hi; ++j) acc += s[j] * (double)v_bh[j * d + c];
#if defined(ORACLE_PLANT_NO_NORMALISE)
    o_row[c] = acc;
#else
    o_row[c] = acc / l;
#endif
  }
#if defined(ORACLE_PLANT_LOG2)
  *lse = m + log2(l);
#elif defined(ORACLE_PLANT_LSE_NO_MAX)
  *lse = log(l);
#else
  *lse = m + log(l);
#endif
}

/* Full or sampled forward.
 *   rows == NULL: every (b, h, i); o has B*H*seq_q*D doubles, lse B*H*seq_q.
 *   rows != NULL: nrows flat row ids r = (b*H + h)*seq_q + i; o has nrows*D, lse nrows.
 * Returns 0, or -1 for invalid sizes or a row id out of range. */
int oracle_attention_fwd(const float* q, const float* k, const float* v, long batch, long heads,
                         long seq_q, long seq_kv, long d, double scale, int causal,
                         const int64_t* rows, long nrows, double* o, double* lse) {
  if (batch < 0 || heads < 0 || seq_q < 0 || seq_kv < 0 || d < 1) return -1;
  long total = batch * heads * seq_q;
  long n = rows ? nrows : total;
  if (rows) {
    for (long t = 0; t < n; ++t)
      if (rows[t] < 0 || rows[t] >= total) return -1;
  }
  int bad = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(seq_kv > 0 ? seq_kv : 1));
    if (!s) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (long t = 0; t < n; ++t) {
      if (!s) continue;
      long r = rows ? (long)rows[t] : t;
      long bh = r / seq_q, i = r % seq_q;
      const float* q_row = q + (size_t)r * d;
      const float* k_bh = k + (size_t)bh * seq_kv * d;
      const float* v_bh = v + (size_t)bh * seq_kv * d;
      long hi = allowed_keys(i, seq_q, seq_kv, causal);
      oracle_row(q_row, k_bh, v_bh, hi, d, seq_kv, scale, s, o + (size_t)t * d, lse + t);
    }
    free(s);
  }
  return bad ? -1 : 0;
}

/* The softmax probabilities of one (batch, head): p[i][j] for i < seq_q, j < seq_kv
 * (zero for keys outside the mask, and whole zero rows where no key is allowed). */
int oracle_attention_probs(const float* q, const float* k, long seq_q, long seq_kv, long d,
                           double scale, int causal, double* p) {
  if (seq_q < 0 || seq_kv < 0 || d < 1) return -1;
  for (long i = 0; i < seq_q; ++i) {
    long hi = allowed_keys(i, seq_q, seq_kv, causal);
    double* row = p + (size_t)i * seq_kv;
    for (long j = 0; j < seq_kv; ++j) row[j] = 0.0;
    if (hi == 0) continue;
    for (long j = 0; j < hi; ++j) {
      double dot = 0.0;
      for (long c = 0; c < d; ++c) dot += (double)q[i * d + c] * (double)k[j * d + c];
      row[j] = scale * dot;
    }
    double m = row[0];
    for (long j = 1; j < hi; ++j)
      if (row[j] > m) m = row[j];
    double l = 0.0;
    for (long j = 0; j < hi; ++j) {
      row[j] = exp(row[j] - m);
      l += row[j];
    }
    for (long j = 0; j < hi; ++j) row[j] /= l;
  }
  return 0;
}

int oracle_num_threads(void) { return omp_get_max_threads(); }
