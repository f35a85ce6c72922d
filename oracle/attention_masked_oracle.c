/* Masked attention-forward oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * The attention forward pass (oxicuda ComputeBackend page, `attention`; the
 * scale multiplies QK^T) with an explicit hard mask: as in the TorchLean
 * page's stable row-wise hard-masked softmax, an entry whose mask value is
 * zero takes no part in the row's max or sum and weighs exactly zero, and a
 * row that admits nothing is all zeros (its log-sum-exp is that of an empty
 * sum, -infinity). Any nonzero mask byte admits. With the causal flag, a key
 * must also satisfy the bottom-right causal bound j <= i + seq_kv - seq_q.
 *
 * Per (b, h) and query row i, with A_i = { j : j <= i + seq_kv - seq_q (causal
 * only) and mask[b, h, i, j] != 0 }:
 *   s_j = scale * q_i . k_j,  m = max_{j in A_i} s_j,  l = sum_{j in A_i} exp(s_j - m),
 *   o_i = sum_{j in A_i} exp(s_j - m) v_j / l,  lse_i = m + log l,
 * all in double, j ascending. Keys outside A_i are never read.
 *
 * Layout: q, o [B][H][seq_q][D]; k, v [B][H][seq_kv][D]; lse [B][H][seq_q];
 * mask bytes, element (b, h, i, j) at mask[b*mask_sb + h*mask_sh + i*seq_kv + j]
 * (a stride of 0 broadcasts the mask over that dimension).
 *
 * Only the tests and the benchmark's CPU baseline use it; the library never
 * does.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>

/* Planted mistakes for the pin tests (MASK_PLANT_*); normal builds define none. */

static int mask_admits(const uint8_t* mrow, long i, long j, long seq_q, long seq_kv, int causal) {
  if (causal && j > i + (seq_kv - seq_q)) {
#if !defined(MASK_PLANT_IGNORE_CAUSAL)
    return 0;
#endif
  }
#if defined(MASK_PLANT_INVERT)
  return mrow[j] == 0;
#else
  return mrow[j] != 0;
#endif
}

int oracle_attention_fwd_masked(const float* q, const float* k, const float* v, const uint8_t* mask,
                                long mask_sb, long mask_sh, long batch, long heads, long seq_q,
                                long seq_kv, long d, double scale, int causal, double* o,
                                double* lse) {
  if (batch < 0 || heads < 0 || seq_q < 0 || seq_kv < 0 || d < 1 || mask_sb < 0 || mask_sh < 0)
    return -1;
  const long nrows = batch * heads * seq_q;
  int bad = 0;
#pragma omp parallel
  {
    long* adm = (long*)malloc(sizeof(long) * (size_t)(seq_kv > 0 ? seq_kv : 1));
    double* s = (double*)malloc(sizeof(double) * (size_t)(seq_kv > 0 ? seq_kv : 1));
    if (!adm || !s) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (long r = 0; r < nrows; ++r) {
      if (!adm || !s) continue;
      const long bh = r / seq_q, i = r % seq_q, b = bh / heads, h = bh % heads;
      const uint8_t* mrow = mask + (size_t)b * mask_sb + (size_t)h * mask_sh + (size_t)i * seq_kv;
      const float* qi = q + (size_t)r * d;
      const float* kb = k + (size_t)bh * seq_kv * d;
      const float* vb = v + (size_t)bh * seq_kv * d;
      double* oi = o + (size_t)r * d;
      long n = 0;
      for (long j = 0; j < seq_kv; ++j)
        if (mask_admits(mrow, i, j, seq_q, seq_kv, causal)) adm[n++] = j;
      if (n == 0) {
        for (long c = 0; c < d; ++c) oi[c] = 0.0;
        lse[r] = -INFINITY;
        continue;
      }
      for (long t = 0; t < n; ++t) {
        double dot = 0.0;
        for (long c = 0; c < d; ++c) dot += (double)qi[c] * (double)kb[(size_t)adm[t] * d + c];
        s[t] = scale * dot;
      }
      double m = s[0];
#if !defined(MASK_PLANT_NO_MAX)
      for (long t = 1; t < n; ++t)
        if (s[t] > m) m = s[t];
#else
      m = 0.0;
#endif
      double l = 0.0;
      for (long t = 0; t < n; ++t) {
        s[t] = exp(s[t] - m);
        l += s[t];
      }
      for (long c = 0; c < d; ++c) {
        double acc = 0.0;
        for (long t = 0; t < n; ++t) acc += s[t] * (double)vb[(size_t)adm[t] * d + c];
        oi[c] = acc / l;
      }
      lse[r] = m + log(l);
    }
    free(adm);
    free(s);
  }
  return bad ? -2 : 0;
}
