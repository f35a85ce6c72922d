/* Masked attention-backward oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * The gradients of the masked attention forward (attention_masked_oracle.c:
 * the oxicuda ComputeBackend `attention` with the TorchLean page's hard
 * mask, a zero mask byte keeping a key out of its row's max and sum, a row
 * that admits nothing all zeros), for an upstream gradient dO = dL/dO.
 *
 * Per (b, h) and query row i, with A_i = { j : j <= i + seq_kv - seq_q
 * (causal only) and mask[b, h, i, j] != 0 }, over j in A_i:
 *   s_ij = scale * q_i . k_j,  P_ij = exp(s_ij - m_i) / sum_{j' in A_i} exp(s_ij' - m_i),
 *   dV_j += P_ij dO_i,  dP_ij = dO_i . v_j,  D_i = sum_{j in A_i} P_ij dP_ij,
 *   dS_ij = P_ij (dP_ij - D_i),  dQ_i = scale sum_j dS_ij k_j,  dK_j += scale dS_ij q_i.
 * The same chain rule as attention_bwd_oracle.c with the prefix of allowed
 * keys replaced by A_i: a blocked pair has no P, so it adds nothing anywhere,
 * and a row with empty A_i has dQ = 0. Everything in double, j ascending,
 * recomputed from q, k, v and dO.
 *
 * The error scale (the _bound function) is that of attention_bwd_oracle.c
 * over the same pairs: each P weighted by 1 + |scale| sum_c |q_ic k_jc| +
 * |lse_i|, every other factor in magnitude.
 *
 * Layout: q, dout, dq [B][H][seq_q][D]; k, v, dk, dv [B][H][seq_kv][D]; mask
 * bytes, element (b, h, i, j) at mask[b*mask_sb + h*mask_sh + i*seq_kv + j]
 * (a stride of 0 broadcasts over that dimension).
 *
 * Only the tests use it; the library never does.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* Planted mistakes for the pin tests (MBWD_PLANT_*); normal builds define none. */

static long masked_set(const uint8_t* mrow, long i, long seq_q, long seq_kv, int causal, long* adm) {
  long n = 0;
  for (long j = 0; j < seq_kv; ++j) {
    if (causal && j > i + (seq_kv - seq_q)) continue;
#if defined(MBWD_PLANT_IGNORE_MASK)
    (void)mrow;
    adm[n++] = j;
#else
    if (mrow[j] != 0) adm[n++] = j;
#endif
  }
  return n;
}

/* P_ij over A_i (n entries at adm) into p; returns lse_i. */
static double masked_probs(const float* qi, const float* kb, long d, double scale, const long* adm,
                           long n, double* p) {
  double m = -INFINITY;
  for (long t = 0; t < n; ++t) {
    double dot = 0.0;
    for (long c = 0; c < d; ++c) dot += (double)qi[c] * (double)kb[(size_t)adm[t] * d + c];
    p[t] = scale * dot;
    if (p[t] > m) m = p[t];
  }
  double l = 0.0;
  for (long t = 0; t < n; ++t) {
    p[t] = exp(p[t] - m);
    l += p[t];
  }
  for (long t = 0; t < n; ++t) p[t] /= l;
  return m + log(l);
}

int oracle_attention_bwd_masked(const float* q, const float* k, const float* v, const float* dout,
                                const uint8_t* mask, long mask_sb, long mask_sh, long batch,
                                long heads, long seq_q, long seq_kv, long d, double scale,
                                int causal, double* dq, double* dk, double* dv) {
  if (batch < 0 || heads < 0 || seq_q < 0 || seq_kv < 0 || d < 1 || mask_sb < 0 || mask_sh < 0)
    return -1;
  const long nbh = batch * heads;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < nbh; ++bh) {
    const long b = bh / heads, h = bh % heads;
    const float* qb = q + (size_t)bh * seq_q * d;
    const float* kb = k + (size_t)bh * seq_kv * d;
    const float* vb = v + (size_t)bh * seq_kv * d;
    const float* gb = dout + (size_t)bh * seq_q * d;
    double* dqb = dq + (size_t)bh * seq_q * d;
    double* dkb = dk + (size_t)bh * seq_kv * d;
    double* dvb = dv + (size_t)bh * seq_kv * d;
    for (size_t e = 0; e < (size_t)seq_q * d; ++e) dqb[e] = 0.0;
    for (size_t e = 0; e < (size_t)seq_kv * d; ++e) dkb[e] = 0.0, dvb[e] = 0.0;
    const size_t nk = (size_t)(seq_kv > 0 ? seq_kv : 1);
    long* adm = (long*)malloc(sizeof(long) * nk);
    double* p = (double*)malloc(sizeof(double) * nk);
    double* ds = (double*)malloc(sizeof(double) * nk);
    if (!adm || !p || !ds) {
#pragma omp atomic write
      bad = 1;
      free(adm);
      free(p);
      free(ds);
      continue;
    }
    for (long i = 0; i < seq_q; ++i) {
      const uint8_t* mrow = mask + (size_t)b * mask_sb + (size_t)h * mask_sh + (size_t)i * seq_kv;
      const long n = masked_set(mrow, i, seq_q, seq_kv, causal, adm);
      if (n == 0) continue;
      const float* qi = qb + (size_t)i * d;
      const float* gi = gb + (size_t)i * d;
      masked_probs(qi, kb, d, scale, adm, n, p);
      double dsum = 0.0;
      for (long t = 0; t < n; ++t) {
        double dp = 0.0;
        for (long c = 0; c < d; ++c) dp += (double)gi[c] * (double)vb[(size_t)adm[t] * d + c];
        ds[t] = dp;
        dsum += p[t] * dp;
      }
      for (long t = 0; t < n; ++t) ds[t] = p[t] * (ds[t] - dsum);
      for (long t = 0; t < n; ++t) {
        const float* kj = kb + (size_t)adm[t] * d;
        double* dkj = dkb + (size_t)adm[t] * d;
        double* dvj = dvb + (size_t)adm[t] * d;
        for (long c = 0; c < d; ++c) {
          dqb[(size_t)i * d + c] += scale * ds[t] * (double)kj[c];
          dkj[c] += scale * ds[t] * (double)qi[c];
          dvj[c] += p[t] * (double)gi[c];
        }
      }
    }
    free(adm);
    free(p);
    free(ds);
  }
  return bad ? -2 : 0;
}

int oracle_attention_bwd_masked_bound(const float* q, const float* k, const float* v,
                                      const float* dout, const uint8_t* mask, long mask_sb,
                                      long mask_sh, long batch, long heads, long seq_q,
                                      long seq_kv, long d, double scale, int causal, double* mq,
                                      double* mk, double* mv) {
  if (batch < 0 || heads < 0 || seq_q < 0 || seq_kv < 0 || d < 1 || mask_sb < 0 || mask_sh < 0)
    return -1;
  const long nbh = batch * heads;
  const double as = fabs(scale);
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < nbh; ++bh) {
    const long b = bh / heads, h = bh % heads;
    const float* qb = q + (size_t)bh * seq_q * d;
    const float* kb = k + (size_t)bh * seq_kv * d;
    const float* vb = v + (size_t)bh * seq_kv * d;
    const float* gb = dout + (size_t)bh * seq_q * d;
    double* mqb = mq + (size_t)bh * seq_q * d;
    double* mkb = mk + (size_t)bh * seq_kv * d;
    double* mvb = mv + (size_t)bh * seq_kv * d;
    for (size_t e = 0; e < (size_t)seq_q * d; ++e) mqb[e] = 0.0;
    for (size_t e = 0; e < (size_t)seq_kv * d; ++e) mkb[e] = 0.0, mvb[e] = 0.0;
    const size_t nk = (size_t)(seq_kv > 0 ? seq_kv : 1);
    long* adm = (long*)malloc(sizeof(long) * nk);
    double* p = (double*)malloc(sizeof(double) * nk);
    double* w = (double*)malloc(sizeof(double) * nk);
    double* pv = (double*)malloc(sizeof(double) * (size_t)d);
    if (!adm || !p || !w || !pv) {
#pragma omp atomic write
      bad = 1;
      free(adm);
      free(p);
      free(w);
      free(pv);
      continue;
    }
    for (long i = 0; i < seq_q; ++i) {
      const uint8_t* mrow = mask + (size_t)b * mask_sb + (size_t)h * mask_sh + (size_t)i * seq_kv;
      const long n = masked_set(mrow, i, seq_q, seq_kv, causal, adm);
      if (n == 0) continue;
      const float* qi = qb + (size_t)i * d;
      const float* gi = gb + (size_t)i * d;
      const double lse = masked_probs(qi, kb, d, scale, adm, n, p);
      for (long t = 0; t < n; ++t) {  /* rho_ij = P_ij (1 + |scale| sum_c |q_ic k_jc| + |lse_i|) */
        double adot = 0.0;
        for (long c = 0; c < d; ++c) adot += fabs((double)qi[c] * (double)kb[(size_t)adm[t] * d + c]);
        p[t] *= 1.0 + as * adot + fabs(lse);
      }
      for (long c = 0; c < d; ++c) pv[c] = 0.0;
      for (long t = 0; t < n; ++t)
        for (long c = 0; c < d; ++c) pv[c] += p[t] * fabs((double)vb[(size_t)adm[t] * d + c]);
      double dmag = 0.0;
      for (long c = 0; c < d; ++c) dmag += fabs((double)gi[c]) * pv[c];
      for (long t = 0; t < n; ++t) {
        double dpm = 0.0;
        for (long c = 0; c < d; ++c) dpm += fabs((double)gi[c] * (double)vb[(size_t)adm[t] * d + c]);
        w[t] = p[t] * (dpm + dmag);
      }
      for (long t = 0; t < n; ++t) {
        const float* kj = kb + (size_t)adm[t] * d;
        double* mkj = mkb + (size_t)adm[t] * d;
        double* mvj = mvb + (size_t)adm[t] * d;
        for (long c = 0; c < d; ++c) {
          mqb[(size_t)i * d + c] += as * w[t] * fabs((double)kj[c]);
          mkj[c] += as * w[t] * fabs((double)qi[c]);
          mvj[c] += p[t] * fabs((double)gi[c]);
        }
      }
    }
    free(adm);
    free(p);
    free(w);
    free(pv);
  }
  return bad ? -2 : 0;
}
