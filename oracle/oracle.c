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

/* gamma_h of the RetNet page ("Multi-Scale Retention (MSR)"): given, or
 * 1 - 2^(-5-h) with 0-based h. */
static double ret_gamma(const double* gamma, int hd) {
  return gamma ? gamma[hd] : 1.0 - ldexp(1.0, -5 - hd);
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
    const double g = ret_gamma(gamma, hd);
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

/*
 * Backward pass of the mLSTM sequence form (vector normaliser, one memory
 * block): the gradients of L = sum_t dh_t . h_t with respect to every input,
 * by the chain rule applied to the recurrence above, one step at a time from
 * t = T-1 down to 0.  Training runs the parallel or chunked forms (section
 * "Triple Paradigm" of the "Edifice.Attention.RetNet" page; the chunked-scan
 * mode of Gdn2Mode on the "burn-gdn2" page); they compute this same function,
 * so its gradient is fixed by the recurrence alone.
 *
 * In true (unstabilised) units, with S_t = f_t S_{t-1} + i_t k_t v_t^T,
 * n_t = f_t n_{t-1} + i_t k_t, z_t = n_t . q_t + bias, h_t = o_t * S_t^T q_t
 * / max(|z_t|, 1), and G_t, g_t the total gradients of L with respect to
 * S_t and n_t (everything from step t on):
 *   G_t = f_{t+1} G_{t+1} + q_t dnum_t^T,  g_t = f_{t+1} g_{t+1} + dz_t q_t,
 *   dnum_t = o_t * dh_t / max(|z_t|, 1),
 *   dz_t = -(o_t * dh_t) . (S_t^T q_t) / max(|z_t|,1)^2 * sign(z_t) when |z_t| > 1, else 0,
 *   dq_t = S_t dnum_t + n_t dz_t,
 *   dk_t = i_t (G_t v_t + g_t),  dv_t = i_t G_t^T k_t,
 *   d i_pre_t = i_t (k_t . G_t v_t + k_t . g_t)           (i = exp(i_pre)),
 *   d log f_t = f_t (<G_t, S_{t-1}> + g_t . n_{t-1}),
 *   d f_pre_t = d log f_t * sigmoid(-f_pre_t)            (log f = log sigmoid(f_pre)),
 *   d o_pre_t = dh_t * (S_t^T q_t / max(|z_t|,1)) * o_t (1 - o_t),
 *   d bias = sum_t dz_t,  dC0 = f_1 G_1 (as gradient of the initial S), dn0 likewise.
 * It runs on the stabilised state: G~_t = e^{m_t} G_t, g~_t = e^{m_t} g_t,
 * which turns the factors above into the f' = e^{lf + m_{t-1} - m_t} and
 * i' = e^{li - m_t} of the forward step and makes dnum, dz use the stabilised
 * denominator max(|z~|, e^{-m}).  The initial-state gradients are returned for
 * the stabilised C0, n0 (d/dC0~ = e^{m0} d/dC0 = f'_1 G~_1).
 *
 * The forward states S~_{t-1}, S~_t are needed at every step; they are
 * recomputed per segment of SEG steps from a saved state at each segment start
 * (checkpoints), so memory stays O((T/SEG + SEG) d_qk d_v).
 *
 * With nb memory blocks (the block-diagonal memory of the "Edifice.Recurrent.
 * XLSTMv2" page, "Key Improvements" item 1) the state and G are block-diagonal
 * [nb][d_qk/nb][d_v/nb]: every product above runs per block, while n~, g and
 * the denominator stay per head.
 * Gradient flowing into the final state (optional): dCT [B,H,nb,d_qk/nb,d_v/nb]
 * and dnT [B,H,d_qk] are the gradients of the loss with respect to the
 * stabilised final state S~_T, n~_T at fixed m_T, i.e. e^{m_T} times the
 * gradients with respect to the true final C_T, n_T.  They start the reverse
 * sweep as G~ and g~ (NULL: zero).  This is the reading under which the
 * downstream loss depends on the final state only through the true state (as
 * a continuation of the recurrence does, its outputs being independent of
 * the stabiliser); no derivative of the stabiliser itself appears.  A second
 * call's dC0, dn0 (for the same m) are exactly the first call's dCT, dnT.
 * dh [B,H,T,d_v] in; outputs (any may be NULL): dq, dk [B,H,T,d_qk]; dv, do_pre
 * [B,H,T,d_v]; di, df [B,H,T]; dbias [H] (summed over B); dbias_t [B,H,T]
 * (the per-token terms dz_t of that sum, in true units); z_t [B,H,T] (the
 * normaliser argument n_t . q_t + bias in true units, whose |.| meets the
 * floor 1 where the gradient jumps); dC0
 * [B,H,nb,d_qk/nb,d_v/nb]; dn0 [B,H,d_qk].  Returns 0, -1 for bad sizes, -2 when out of memory.
 */
int oracle_mlstm_bwd(int B, int H, int T, int dqk, int dv, int nb, const double* q,
                     const double* k, const double* v, const double* i_pre,
                     const double* f_pre, const double* o_pre, const double* bias,
                     const double* C0, const double* n0, const double* m0,
                     const double* dh, const double* dCT, const double* dnT,
                     double* dq, double* dk, double* dvo,
                     double* di, double* df, double* do_pre, double* dbias,
                     double* dbias_t, double* z_t, double* dC0, double* dn0) {
  if (B < 0 || H < 0 || T < 0 || dqk <= 0 || dv <= 0 || nb <= 0) return -1;
  if (dqk % nb || dv % nb) return -1;
  const int dqkb = dqk / nb, dvb = dv / nb;
  const size_t csz = (size_t)dqk * dv / nb; /* [nb][dqkb][dvb] */
  const size_t ssz = csz + (size_t)dqk + 1; /* one saved state: S~, n~, m */
  const long BH = (long)B * H;
  int SEG = 1;
  while ((long)SEG * SEG < T) ++SEG;
  const int NSEG = T > 0 ? (T + SEG - 1) / SEG : 0;
  double* dbias_bh = (double*)calloc(BH > 0 ? (size_t)BH : 1, sizeof(double));
  if (!dbias_bh) return -2;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    const int hd = (int)(bh % H);
    const double bs = bias ? bias[hd] : 0.0;
    /* ckpt[s]: state before segment s; seg[j]: state after step s*SEG + j */
    double* ckpt = (double*)malloc((size_t)(NSEG + 1) * ssz * sizeof(double));
    double* seg = (double*)malloc((size_t)(SEG + 1) * ssz * sizeof(double));
    double* G = (double*)calloc(csz, sizeof(double));
    double* g = (double*)calloc((size_t)dqk, sizeof(double));
    double* hbuf = (double*)malloc((size_t)dv * sizeof(double));
    double* dn = (double*)malloc((size_t)dv * sizeof(double));
    double* Gv = (double*)malloc((size_t)dqk * sizeof(double));
    if (!ckpt || !seg || !G || !g || !hbuf || !dn || !Gv) {
      free(ckpt), free(seg), free(G), free(g), free(hbuf), free(dn), free(Gv);
#pragma omp atomic write
      bad = 1;
      continue;
    }
    /* the gradient arriving at the final state */
    if (dCT) memcpy(G, dCT + bh * csz, csz * sizeof(double));
    if (dnT) memcpy(g, dnT + bh * dqk, (size_t)dqk * sizeof(double));
    /* forward sweep: the state at every segment start */
    double* s0 = ckpt;
    if (C0) memcpy(s0, C0 + bh * csz, csz * sizeof(double));
    else memset(s0, 0, csz * sizeof(double));
    if (n0) memcpy(s0 + csz, n0 + bh * dqk, (size_t)dqk * sizeof(double));
    else memset(s0 + csz, 0, (size_t)dqk * sizeof(double));
    s0[csz + dqk] = m0 ? m0[bh] : 0.0;
    for (int s = 0; s < NSEG; ++s) {
      double* cur = ckpt + (size_t)(s + 1) * ssz;
      memcpy(cur, ckpt + (size_t)s * ssz, ssz * sizeof(double));
      for (int t = s * SEG; t < T && t < (s + 1) * SEG; ++t) {
        const size_t tok = (size_t)bh * T + t;
        cell_step(dqk, dv, nb, q + tok * dqk, k + tok * dqk, v + tok * dv, i_pre[tok],
                  f_pre[tok], o_pre ? o_pre + tok * dv : NULL, bs, 1, 0.0, cur,
                  cur + csz, cur + csz + dqk, hbuf);
      }
    }
    double dbias_acc = 0.0;
    for (int s = NSEG - 1; s >= 0; --s) {
      /* recompute the segment: seg[0] = state before it, seg[j+1] after step j */
      const int t0 = s * SEG, t1 = (s + 1) * SEG < T ? (s + 1) * SEG : T;
      memcpy(seg, ckpt + (size_t)s * ssz, ssz * sizeof(double));
      for (int t = t0; t < t1; ++t) {
        const size_t tok = (size_t)bh * T + t;
        double* nxt = seg + (size_t)(t - t0 + 1) * ssz;
        memcpy(nxt, seg + (size_t)(t - t0) * ssz, ssz * sizeof(double));
        cell_step(dqk, dv, nb, q + tok * dqk, k + tok * dqk, v + tok * dv, i_pre[tok],
                  f_pre[tok], o_pre ? o_pre + tok * dv : NULL, bs, 1, 0.0, nxt,
                  nxt + csz, nxt + csz + dqk, hbuf);
      }
      for (int t = t1 - 1; t >= t0; --t) {
        const size_t tok = (size_t)bh * T + t;
        const double* Sp = seg + (size_t)(t - t0) * ssz; /* S~_{t-1}, n~_{t-1}, m_{t-1} */
        const double* St = Sp + ssz;                     /* S~_t, n~_t, m_t */
        const double* np_ = Sp + csz;
        const double* nt = St + csz;
        const double mp = Sp[csz + dqk], mt = St[csz + dqk];
        const double* qt = q + tok * dqk;
        const double* kt = k + tok * dqk;
        const double* vt = v + tok * dv;
        const double* dht = dh + tok * dv;
        /* readout at t on the updated state */
        double zt = 0.0;
        for (int r = 0; r < dqk; ++r) zt += nt[r] * qt[r];
        const double fl = exp(-mt);
        zt += bs * fl;
        const double den = fmax(fabs(zt), fl);
        double sdy = 0.0; /* (o * dh) . y */
        for (int c = 0; c < dv; ++c) {
          const int b = c / dvb, cc = c % dvb;
          const double* Sb = St + (size_t)b * dqkb * dvb;
          double num = 0.0;
          for (int r = 0; r < dqkb; ++r) num += Sb[(size_t)r * dvb + cc] * qt[b * dqkb + r];
          const double y = num / den;
          const double o = o_pre ? sigmoid(o_pre[tok * dv + c]) : 1.0;
          if (do_pre && o_pre) do_pre[tok * dv + c] = dht[c] * y * o * (1.0 - o);
          dn[c] = o * dht[c] / den;
          sdy += o * dht[c] * y;
        }
        const double dz = fabs(zt) > fl ? -sdy / den * (zt > 0 ? 1.0 : -1.0) : 0.0;
        dbias_acc += dz * fl;
        if (dbias_t) dbias_t[tok] = dz * fl;
        if (z_t) z_t[tok] = zt / fl;
        /* dq_t = S~_t dn + n~_t dz (the matrix per block, n~ over the head) */
        if (dq)
          for (int d = 0; d < dqk; ++d) {
            const int b = d / dqkb, r = d % dqkb;
            const double* Sr = St + (size_t)b * dqkb * dvb + (size_t)r * dvb;
            double a = nt[d] * dz;
            for (int cc = 0; cc < dvb; ++cc) a += Sr[cc] * dn[b * dvb + cc];
            dq[tok * dqk + d] = a;
          }
        /* total gradients of the state at t (block-diagonal, like the state) */
        for (int d = 0; d < dqk; ++d) {
          const int b = d / dqkb, r = d % dqkb;
          double* Gr = G + (size_t)b * dqkb * dvb + (size_t)r * dvb;
          for (int cc = 0; cc < dvb; ++cc) Gr[cc] += qt[d] * dn[b * dvb + cc];
          g[d] += qt[d] * dz;
        }
        /* through S~_t = f' S~_{t-1} + i' k v^T (per block) */
        const double lf = log_sigmoid(f_pre[tok]);
        const double fdec = exp(lf + mp - mt), iw = exp(i_pre[tok] - mt);
        double kGv = 0.0, kg = 0.0, dlf = 0.0;
        for (int d = 0; d < dqk; ++d) {
          const int b = d / dqkb, r = d % dqkb;
          const size_t ro = (size_t)b * dqkb * dvb + (size_t)r * dvb;
          double a = 0.0, bb = np_[d] * g[d];
          for (int cc = 0; cc < dvb; ++cc) {
            a += G[ro + cc] * vt[b * dvb + cc];
            bb += G[ro + cc] * Sp[ro + cc];
          }
          Gv[d] = a;
          kGv += kt[d] * a;
          kg += kt[d] * g[d];
          dlf += bb;
        }
        dlf *= fdec;
        if (dk)
          for (int d = 0; d < dqk; ++d) dk[tok * dqk + d] = iw * (Gv[d] + g[d]);
        if (dvo)
          for (int c = 0; c < dv; ++c) {
            const int b = c / dvb, cc = c % dvb;
            double a = 0.0;
            for (int r = 0; r < dqkb; ++r) a += G[(size_t)b * dqkb * dvb + (size_t)r * dvb + cc] * kt[b * dqkb + r];
            dvo[tok * dv + c] = iw * a;
          }
        if (di) di[tok] = iw * (kGv + kg);
        if (df) df[tok] = dlf * sigmoid(-f_pre[tok]);
        /* on to step t-1: G~_{t-1} = f' G~_t */
        for (size_t e = 0; e < csz; ++e) G[e] *= fdec;
        for (int r = 0; r < dqk; ++r) g[r] *= fdec;
      }
    }
    if (dC0) memcpy(dC0 + bh * csz, G, csz * sizeof(double));
    if (dn0) memcpy(dn0 + bh * dqk, g, (size_t)dqk * sizeof(double));
    dbias_bh[bh] = dbias_acc;
    free(ckpt), free(seg), free(G), free(g), free(hbuf), free(dn), free(Gv);
  }
  if (dbias)
    for (int hd = 0; hd < H; ++hd) {
      double a = 0.0;
      for (int b = 0; b < B; ++b) a += dbias_bh[(long)b * H + hd];
      dbias[hd] = a;
    }
  free(dbias_bh);
  return bad ? -2 : 0;
}

/*
 * Backward pass of retention (recurrent form above): the gradients of
 * L = sum_t dout_t . out_t.  With G_t the total gradient of L with respect to
 * the state after token t,
 *   G_t = gamma G_{t+1} + q_t dout_t^T,
 *   dq_t = S_t dout_t,  dk_t = G_t v_t,  dv_t = G_t^T k_t,
 *   dS0 = gamma G_0 (gradient of the initial state).
 * dq comes from a forward sweep over the states, dk, dv, dS0 from a reverse
 * sweep over G.  gamma may be NULL (1 - 2^(-5-h)); S0 may be NULL (zero).
 * Outputs may be NULL.  Returns 0, -1 for bad sizes, -2 when out of memory.
 */
int oracle_retention_bwd(int B, int H, int T, int dk, int dv, const double* q,
                         const double* k, const double* v, const double* gamma,
                         const double* S0, const double* dout, const double* dST,
                         double* dq, double* dk_out, double* dv_out, double* dS0) {
  if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
  const size_t ssz = (size_t)dk * dv;
  const long BH = (long)B * H;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    const int hd = (int)(bh % H);
    const double g = ret_gamma(gamma, hd);
    double* S = (double*)malloc(ssz * sizeof(double));
    if (!S) {
#pragma omp atomic write
      bad = 1;
      continue;
    }
    /* forward sweep: S_t, dq_t = S_t dout_t */
    if (S0) memcpy(S, S0 + bh * ssz, ssz * sizeof(double));
    else memset(S, 0, ssz * sizeof(double));
    for (int t = 0; t < T; ++t) {
      const size_t tok = (size_t)bh * T + t;
      const double* kt = k + tok * dk;
      const double* vt = v + tok * dv;
      const double* gt = dout + tok * dv;
      for (int r = 0; r < dk; ++r)
        for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] = kt[r] * vt[c] + g * S[(size_t)r * dv + c];
      if (dq)
        for (int r = 0; r < dk; ++r) {
          double a = 0.0;
          for (int c = 0; c < dv; ++c) a += S[(size_t)r * dv + c] * gt[c];
          dq[tok * dk + r] = a;
        }
    }
    /* reverse sweep: G_t = gamma G_{t+1} + q_t dout_t^T (S reused as G),
     * starting from the gradient arriving at the final state, G_{T-1} =
     * dS_T + q_{T-1} dout_{T-1}^T */
    if (dST) memcpy(S, dST + bh * ssz, ssz * sizeof(double));
    else memset(S, 0, ssz * sizeof(double));
    for (int t = T - 1; t >= 0; --t) {
      const size_t tok = (size_t)bh * T + t;
      const double* qt = q + tok * dk;
      const double* kt = k + tok * dk;
      const double* vt = v + tok * dv;
      const double* gt = dout + tok * dv;
      const double gd = t == T - 1 ? 1.0 : g; /* G_{t+1} decays into G_t */
      for (int r = 0; r < dk; ++r)
        for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] = gd * S[(size_t)r * dv + c] + qt[r] * gt[c];
      if (dk_out)
        for (int r = 0; r < dk; ++r) {
          double a = 0.0;
          for (int c = 0; c < dv; ++c) a += S[(size_t)r * dv + c] * vt[c];
          dk_out[tok * dk + r] = a;
        }
      if (dv_out)
        for (int c = 0; c < dv; ++c) {
          double a = 0.0;
          for (int r = 0; r < dk; ++r) a += S[(size_t)r * dv + c] * kt[r];
          dv_out[tok * dv + c] = a;
        }
    }
    if (dS0)
      for (size_t e = 0; e < ssz; ++e) dS0[bh * ssz + e] = g * S[e];
    free(S);
  }
  return bad ? -2 : 0;
}
