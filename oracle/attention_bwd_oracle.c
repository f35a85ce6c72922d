/* Attention-backward oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain double-precision CPU statement of the gradients of the attention
 * forward pass (oxicuda ComputeBackend page, `attention`; scale read as a
 * multiplier of QK^T; bottom-right causal mask; rows with no allowed key all
 * zeros). Only the tests use it; the library never links or calls it.
 *
 * For a loss L with upstream gradient dO = dL/dO, per (batch, head), over
 * the allowed pairs (i, j) (j < hi(i)):
 *
 *   s_ij  = scale * q_i . k_j
 *   P_ij  = exp(s_ij - m_i) / sum_j' exp(s_ij' - m_i)      (the forward's softmax)
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   D_i   = sum_j P_ij dP_ij                              (= dO_i . O_i)
 *   dS_ij = P_ij (dP_ij - D_i)                            (softmax Jacobian)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 *
 * Everything is recomputed from q, k, v and dO; nothing is taken from a
 * forward pass. Rows with no allowed key have P = 0 and contribute nothing.
 * The pages name a softmax backward (pulsatrix `softmax_rows_backward`,
 * MicroGPT `fused_attn_softmax_backward`); the formula above is that
 * Jacobian-vector product composed with the two products of the forward.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdlib.h>

/* Planted mistakes for the pin tests (BWD_PLANT_*); normal builds define none. */

static long bwd_allowed(long i, long seq_q, long seq_kv, int causal) {
  if (!causal) return seq_kv;
#if defined(BWD_PLANT_TOP_LEFT)
  long hi = i + 1;
#else
  long hi = i + (seq_kv - seq_q) + 1;
#endif
  if (hi < 0) hi = 0;
  if (hi > seq_kv) hi = seq_kv;
  return hi;
}

int oracle_attention_bwd(const float* q, const float* k, const float* v, const float* dout,
                         long batch, long heads, long seq_q, long seq_kv, long d, double scale,
                         int causal, double* dq, double* dk, double* dv) {
  if (batch < 0 || heads < 0 || seq_q < 0 || seq_kv < 0 || d < 1) return -1;
  const long nbh = batch * heads;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < nbh; ++bh) {
    const float* qb = q + (size_t)bh * seq_q * d;
    const float* kb = k + (size_t)bh * seq_kv * d;
    const float* vb = v + (size_t)bh * seq_kv * d;
    const float* gb = dout + (size_t)bh * seq_q * d;
    double* dqb = dq + (size_t)bh * seq_q * d;
    double* dkb = dk + (size_t)bh * seq_kv * d;
    double* dvb = dv + (size_t)bh * seq_kv * d;
    for (size_t e = 0; e < (size_t)seq_q * d; ++e) dqb[e] = 0.0;
    for (size_t e = 0; e < (size_t)seq_kv * d; ++e) dkb[e] = 0.0, dvb[e] = 0.0;
    double* p = (double*)malloc(sizeof(double) * (seq_kv > 0 ? seq_kv : 1));
    double* ds = (double*)malloc(sizeof(double) * (seq_kv > 0 ? seq_kv : 1));
    if (!p || !ds) {
#pragma omp atomic write
      bad = 1;
      free(p);
      free(ds);
      continue;
    }
    for (long i = 0; i < seq_q; ++i) {
      const long hi = bwd_allowed(i, seq_q, seq_kv, causal);
      if (hi == 0) continue;
      const float* qi = qb + (size_t)i * d;
      const float* gi = gb + (size_t)i * d;
      double m = -INFINITY;
      for (long j = 0; j < hi; ++j) {
        double dot = 0.0;
        for (long c = 0; c < d; ++c) dot += (double)qi[c] * (double)kb[(size_t)j * d + c];
        p[j] = scale * dot;
        if (p[j] > m) m = p[j];
      }
      double l = 0.0;
      for (long j = 0; j < hi; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
      }
      for (long j = 0; j < hi; ++j) p[j] /= l;
      double dsum = 0.0;
      for (long j = 0; j < hi; ++j) {
        double dp = 0.0;
        for (long c = 0; c < d; ++c) dp += (double)gi[c] * (double)vb[(size_t)j * d + c];
        ds[j] = dp;
        dsum += p[j] * dp;
      }
      for (long j = 0; j < hi; ++j) {
#if defined(BWD_PLANT_NO_D)
        ds[j] = p[j] * ds[j];
#else
        ds[j] = p[j] * (ds[j] - dsum);
#endif
      }
      for (long j = 0; j < hi; ++j) {
        const float* kj = kb + (size_t)j * d;
        double* dkj = dkb + (size_t)j * d;
        double* dvj = dvb + (size_t)j * d;
        for (long c = 0; c < d; ++c) {
          dqb[(size_t)i * d + c] += scale * ds[j] * (double)kj[c];
#if defined(BWD_PLANT_NO_SCALE_DK)
          dkj[c] += ds[j] * (double)qi[c];
#else
          dkj[c] += scale * ds[j] * (double)qi[c];
#endif
#if defined(BWD_PLANT_DV_USES_DS)
          dvj[c] += ds[j] * (double)gi[c];
#else
          dvj[c] += p[j] * (double)gi[c];
#endif
        }
      }
    }
    free(p);
    free(ds);
  }
  return bad ? -2 : 0;
}

/* Error scale of the gradients, for the parity tolerance: the sums of
 * oracle_attention_bwd with every factor replaced by its magnitude, and each
 * probability weighted by the size of its exponent's terms. exp(x) computed
 * from an argument carrying an absolute error of e|x|-ish has a relative error
 * of that order, so P_ij counts as rho_ij = P_ij (1 + a_ij) with
 * a_ij = |scale| sum_c |q_ic k_jc| + |lse_i|. With
 * dPmag_ij = sum_c |dO_ic v_jc| and Dmag_i = sum_c |dO_ic| sum_j rho_ij |v_jc|
 * (bounds of |dP_ij| and of |D_i|, also of D formed from a rounded O):
 *   mv_j = sum_i rho_ij |dO_i|
 *   mk_j = |scale| sum_i rho_ij (dPmag_ij + Dmag_i) |q_i|
 *   mq_i = |scale| sum_j rho_ij (dPmag_ij + Dmag_i) |k_j|
 * A computed gradient whose every term carries a relative error of at most e
 * (relative to these weights) is off by at most e times them, elementwise; by
 * the triangle inequality they also bound |dv|, |dk| and |dq|. */
int oracle_attention_bwd_bound(const float* q, const float* k, const float* v, const float* dout,
                               long batch, long heads, long seq_q, long seq_kv, long d,
                               double scale, int causal, double* mq, double* mk, double* mv) {
  if (batch < 0 || heads < 0 || seq_q < 0 || seq_kv < 0 || d < 1) return -1;
  const long nbh = batch * heads;
  const double as = fabs(scale);
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < nbh; ++bh) {
    const float* qb = q + (size_t)bh * seq_q * d;
    const float* kb = k + (size_t)bh * seq_kv * d;
    const float* vb = v + (size_t)bh * seq_kv * d;
    const float* gb = dout + (size_t)bh * seq_q * d;
    double* mqb = mq + (size_t)bh * seq_q * d;
    double* mkb = mk + (size_t)bh * seq_kv * d;
    double* mvb = mv + (size_t)bh * seq_kv * d;
    for (size_t e = 0; e < (size_t)seq_q * d; ++e) mqb[e] = 0.0;
    for (size_t e = 0; e < (size_t)seq_kv * d; ++e) mkb[e] = 0.0, mvb[e] = 0.0;
    double* p = (double*)malloc(sizeof(double) * (seq_kv > 0 ? seq_kv : 1));
    double* sa = (double*)malloc(sizeof(double) * (seq_kv > 0 ? seq_kv : 1));
    double* w = (double*)malloc(sizeof(double) * (seq_kv > 0 ? seq_kv : 1));
    double* pv = (double*)malloc(sizeof(double) * d);
    if (!p || !sa || !w || !pv) {
#pragma omp atomic write
      bad = 1;
      free(p);
      free(sa);
      free(w);
      free(pv);
      continue;
    }
    for (long i = 0; i < seq_q; ++i) {
      const long hi = bwd_allowed(i, seq_q, seq_kv, causal);
      if (hi == 0) continue;
      const float* qi = qb + (size_t)i * d;
      const float* gi = gb + (size_t)i * d;
      double m = -INFINITY;
      for (long j = 0; j < hi; ++j) {
        double dot = 0.0, adot = 0.0;
        for (long c = 0; c < d; ++c) {
          const double t = (double)qi[c] * (double)kb[(size_t)j * d + c];
          dot += t;
          adot += fabs(t);
        }
        p[j] = scale * dot;
        sa[j] = as * adot;
        if (p[j] > m) m = p[j];
      }
      double l = 0.0;
      for (long j = 0; j < hi; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
      }
      const double lse = m + log(l);
      for (long j = 0; j < hi; ++j) p[j] = p[j] / l * (1.0 + sa[j] + fabs(lse));  /* rho_ij */
      for (long c = 0; c < d; ++c) pv[c] = 0.0;
      for (long j = 0; j < hi; ++j)
        for (long c = 0; c < d; ++c) pv[c] += p[j] * fabs((double)vb[(size_t)j * d + c]);
      double dmag = 0.0;
      for (long c = 0; c < d; ++c) dmag += fabs((double)gi[c]) * pv[c];
      for (long j = 0; j < hi; ++j) {
        double dpm = 0.0;
        for (long c = 0; c < d; ++c) dpm += fabs((double)gi[c] * (double)vb[(size_t)j * d + c]);
        w[j] = p[j] * (dpm + dmag);
      }
      for (long j = 0; j < hi; ++j) {
        const float* kj = kb + (size_t)j * d;
        double* mkj = mkb + (size_t)j * d;
        double* mvj = mvb + (size_t)j * d;
        for (long c = 0; c < d; ++c) {
          mqb[(size_t)i * d + c] += as * w[j] * fabs((double)kj[c]);
          mkj[c] += as * w[j] * fabs((double)qi[c]);
          mvj[c] += p[j] * fabs((double)gi[c]);
        }
      }
    }
    free(p);
    free(sa);
    free(w);
    free(pv);
  }
  return bad ? -2 : 0;
}
