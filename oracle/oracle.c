/*
 * Plain fp64 CPU oracle for the mLSTM matrix-memory recurrence and for
 * RetNet retention.  TEST INFRASTRUCTURE ONLY: the tests, the package's smoke
 * check and the benchmark's CPU-baseline leg call it; the GPU library never
 * links, loads or calls it, and it includes no header of the GPU library.
 *
 * What it computes (sources):
 *  - Matrix memory update C_t = f_t C_{t-1} + i_t (v_t (x) k_t):
 *    "mLSTM Model" page (DeepChrInteract-v2), section "Core idea", display math.
 *  - "gating is stabilized in log space": same page and section.  The page
 *    gives no rule; this oracle uses the max stabiliser
 *    m_t = max(log f_t + m_{t-1}, log i_t) with m_0 = 0 (plain reading).
 *  - Exponential input gate i = exp(i_pre), sigmoid forget gate
 *    f = sigmoid(f_pre), sigmoid output gate o = sigmoid(o_pre), vector
 *    normaliser n_t = f n_{t-1} + i k_t and readout
 *    h_t = o_t * (C_t q_t) / max(|n_t . q_t + bias|, 1): the xLSTM cell of
 *    Beck et al. that the "Edifice.Recurrent.XLSTMv2" page cites under
 *    "References", with the learnable normaliser bias of that page's
 *    "Key Improvements over xLSTM v1", item 2.  That item prints a scalar
 *    normaliser without the query; the vector reading n . q is used here.
 *  - Block-diagonal memory: same page, "Key Improvements", item 1.  Only the
 *    matrix is split into independent blocks (q, k, v split into nb contiguous
 *    slices); gates, stabiliser, the full-length normaliser and the
 *    denominator stay per head.
 *  - Retention recurrence s_n = gamma s_{n-1} + K_n^T V_n, o_n = Q_n s_n and
 *    gamma_h = 1 - 2^(-5-h): "Edifice.Attention.RetNet" page, sections
 *    "Key Innovation: Retention Mechanism" and "Multi-Scale Retention (MSR)".
 *
 * Representation.  The state is kept stabilised: S~ = C^T e^{-m} stored
 * [d_qk][d_v] (v index fastest, the [B,H,K,V] layout of the "burn-gdn2"
 * Gdn2Mode::FusedRecurrent doc and of init_retention_state on the RetNet
 * page), n~ = n e^{-m}.  Dividing numerator and denominator of the readout by
 * e^{m_t} gives h_t = o_t * (S~^T q_t) / max(|n~ . q_t + bias e^{-m_t}|, e^{-m_t}),
 * which equals the unstabilised readout exactly.
 *
 * Layouts (row-major, contiguous, fp64):
 *   q, k [B,H,T,d_qk]; v, o_pre, h [B,H,T,d_v]; i_pre, f_pre [B,H,T];
 *   bias [H]; C [B,H,nb,d_qk/nb,d_v/nb]; n [B,H,d_qk]; m [B,H].
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* log(sigmoid(x)) without overflow. */
static double log_sigmoid(double x) {
  if (x >= 0.0) return -log1p(exp(-x));
  return x - log1p(exp(x));
}

static double sigmoid(double x) {
  if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
  double e = exp(x);
  return e / (1.0 + e);
}

/*
 * One time step of one (batch, head) cell, in place on (S, n, m).
 * S: [nb][dqkb][dvb]; n: [dqk]; *m: scalar.  Writes h[dv].
 * shift: extra amount added to the stabiliser after the max rule (0 for the
 * plain oracle; the shift-invariance test passes non-zero values).
 * normalise selects the normaliser:
 *   0  none: the retention special case h = o * S~^T q;
 *   1  vector n~ = f' n~ + i' k, denominator |n~ . q + bias e^{-m}| per head
 *      (the reading used throughout);
 *   2  scalar n~ = f' n~ + i' kept in n[0], denominator |n~ + bias e^{-m}|:
 *      the normaliser exactly as the "Edifice.Recurrent.XLSTMv2" page prints
 *      it in "Key Improvements over xLSTM v1", item 2 (no k, no q);
 *   3  vector n~ as in 1, but each memory block divides by its own
 *      |n~_beta . q_beta + bias e^{-m}| (a per-block normaliser for the
 *      block-diagonal memory of item 1).
 * The floor max(., e^{-m}) is the page's max(., 1) in stabilised units.
 */
static void cell_step(int dqk, int dv, int nb, const double* q, const double* k,
                      const double* v, double i_pre, double f_pre,
                      const double* o_pre, double bias, int normalise,
                      double shift, double* S, double* n, double* m,
                      double* h) {
  const int dqkb = dqk / nb, dvb = dv / nb;
  const double lf = log_sigmoid(f_pre);
  const double li = i_pre;
  double m_new = fmax(lf + *m, li) + shift;
  const double fdec = exp(lf + *m - m_new);
  const double iw = exp(li - m_new);
  /* S~_beta = f' S~_beta + i' k_beta v_beta^T, per block. */
  for (int b = 0; b < nb; ++b) {
    double* Sb = S + (size_t)b * dqkb * dvb;
    const double* kb = k + (size_t)b * dqkb;
    const double* vb = v + (size_t)b * dvb;
    for (int r = 0; r < dqkb; ++r)
      for (int c = 0; c < dvb; ++c)
        Sb[(size_t)r * dvb + c] = fdec * Sb[(size_t)r * dvb + c] + iw * kb[r] * vb[c];
  }
  /* n~ = f' n~ + i' k (full head), or the scalar n~ = f' n~ + i'. */
  if (normalise == 2) n[0] = fdec * n[0] + iw;
  else
    for (int r = 0; r < dqk; ++r) n[r] = fdec * n[r] + iw * k[r];
  /* Readout with the updated state: num_beta = S~_beta^T q_beta. */
  double den = 0.0;
  if (normalise == 2) den = n[0];
  else
    for (int r = 0; r < dqk; ++r) den += n[r] * q[r];
  const double floor_ = exp(-m_new);
  double denom = fmax(fabs(den + bias * floor_), floor_);
  for (int b = 0; b < nb; ++b) {
    const double* Sb = S + (size_t)b * dqkb * dvb;
    const double* qb = q + (size_t)b * dqkb;
    if (normalise == 3) {
      double db = 0.0;
      for (int r = 0; r < dqkb; ++r) db += n[(size_t)b * dqkb + r] * qb[r];
      denom = fmax(fabs(db + bias * floor_), floor_);
    }
    for (int c = 0; c < dvb; ++c) {
      double num = 0.0;
      for (int r = 0; r < dqkb; ++r) num += Sb[(size_t)r * dvb + c] * qb[r];
      const double o = o_pre ? sigmoid(o_pre[(size_t)b * dvb + c]) : 1.0;
      h[(size_t)b * dvb + c] = normalise ? o * num / denom : o * num;
    }
  }
  *m = m_new;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Sequence form: a plain loop over t = 1..T for every (b, h).
 * C0/n0/m0 may be NULL (zero state, m = 0).  C_out/n_out/m_out may be NULL.
 * m_shift [B,H,T] may be NULL.  normalise: 1 for mLSTM, 0 for "no normaliser".
 * Returns 0, or -1 for bad sizes.
 */
int oracle_mlstm_fwd(int B, int H, int T, int dqk, int dv, int nb, int normalise,
                     const double* q, const double* k, const double* v,
                     const double* i_pre, const double* f_pre,
                     const double* o_pre, const double* bias,
                     const double* C0, const double* n0, const double* m0,
                     const double* m_shift, double* h, double* C_out,
                     double* n_out, double* m_out) {
  if (B < 0 || H < 0 || T < 0 || dqk <= 0 || dv <= 0 || nb <= 0) return -1;
  if (dqk % nb || dv % nb) return -1;
  const size_t csz = (size_t)dqk * dv / nb;
  const long BH = (long)B * H;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    const int hd = (int)(bh % H);
    double* S = (double*)malloc(csz * sizeof(double));
    double* n = (double*)malloc((size_t)dqk * sizeof(double));
    if (!S || !n) {
      free(S);
      free(n);
#pragma omp atomic write
      bad = 1;
      continue;
    }
    if (C0) memcpy(S, C0 + bh * csz, csz * sizeof(double));
    else memset(S, 0, csz * sizeof(double));
    if (n0) memcpy(n, n0 + bh * dqk, (size_t)dqk * sizeof(double));
    else memset(n, 0, (size_t)dqk * sizeof(double));
    double m = m0 ? m0[bh] : 0.0;
    const double bs = bias ? bias[hd] : 0.0;
    for (int t = 0; t < T; ++t) {
      const size_t tok = (size_t)bh * T + t;
      cell_step(dqk, dv, nb, q + tok * dqk, k + tok * dqk, v + tok * dv,
                i_pre[tok], f_pre[tok], o_pre ? o_pre + tok * dv : NULL, bs,
                normalise, m_shift ? m_shift[tok] : 0.0, S, n, &m,
                h + tok * dv);
    }
    if (C_out) memcpy(C_out + bh * csz, S, csz * sizeof(double));
    if (n_out) memcpy(n_out + bh * dqk, n, (size_t)dqk * sizeof(double));
    if (m_out) m_out[bh] = m;
    free(S);
    free(n);
  }
  return bad ? -2 : 0;
}

/*
 * Single-token decode step on every (b, h), state updated in place
 * (the in-place carried state of the burn-gdn2 Gdn2Mode::FusedRecurrent doc).
 * q,k [B,H,dqk]; v,o_pre,h [B,H,dv]; i_pre,f_pre [B,H]; C,n,m as above.
 */
int oracle_mlstm_step(int B, int H, int dqk, int dv, int nb, int normalise,
                      const double* q, const double* k, const double* v,
                      const double* i_pre, const double* f_pre,
                      const double* o_pre, const double* bias, double* C,
                      double* n, double* m, double* h) {
  if (B < 0 || H < 0 || dqk <= 0 || dv <= 0 || nb <= 0) return -1;
  if (dqk % nb || dv % nb) return -1;
  const size_t csz = (size_t)dqk * dv / nb;
  const long BH = (long)B * H;
#pragma omp parallel for schedule(static)
  for (long bh = 0; bh < BH; ++bh) {
    const int hd = (int)(bh % H);
    cell_step(dqk, dv, nb, q + bh * dqk, k + bh * dqk, v + bh * dv, i_pre[bh],
              f_pre[bh], o_pre ? o_pre + bh * dv : NULL, bias ? bias[hd] : 0.0,
              normalise, 0.0, C + bh * csz, n + bh * dqk, m + bh, h + bh * dv);
  }
  return 0;
}

/*
 * Retention, recurrent form: s = gamma_h s + k v^T; out = s^T q, for every
 * (b, h) and t.  gamma may be NULL: then gamma_h = 1 - 2^(-5-h), h = 0..H-1.
 * q,k [B,H,T,dk]; v,out [B,H,T,dv]; S0/S_out [B,H,dk,dv] (may be NULL).
 */
int oracle_retention_fwd(int B, int H, int T, int dk, int dv, const double* q,
                         const double* k, const double* v, const double* gamma,
                         const double* S0, double* out, double* S_out) {
  if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
  const size_t ssz = (size_t)dk * dv;
  const long BH = (long)B * H;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    const int hd = (int)(bh % H);
    const double g = gamma ? gamma[hd] : 1.0 - ldexp(1.0, -5 - hd);
    double* S = (double*)malloc(ssz * sizeof(double));
    if (!S) {
#pragma omp atomic write
      bad = 1;
      continue;
    }
    if (S0) memcpy(S, S0 + bh * ssz, ssz * sizeof(double));
    else memset(S, 0, ssz * sizeof(double));
    for (int t = 0; t < T; ++t) {
      const size_t tok = (size_t)bh * T + t;
      const double* qt = q + tok * dk;
      const double* kt = k + tok * dk;
      const double* vt = v + tok * dv;
      for (int r = 0; r < dk; ++r)
        for (int c = 0; c < dv; ++c)
          S[(size_t)r * dv + c] = g * S[(size_t)r * dv + c] + kt[r] * vt[c];
      double* ot = out + tok * dv;
      for (int c = 0; c < dv; ++c) {
        double acc = 0.0;
        for (int r = 0; r < dk; ++r) acc += S[(size_t)r * dv + c] * qt[r];
        ot[c] = acc;
      }
    }
    if (S_out) memcpy(S_out + bh * ssz, S, ssz * sizeof(double));
    free(S);
  }
  return bad ? -2 : 0;
}
