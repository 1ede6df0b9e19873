"""fp64 numpy model of the chunkwise algorithm that the HIP kernels implement.

It is not the oracle: it is the kernel's algebra written out plainly so that
the CPU tests can check, before and independently of any GPU code, that the
chunk / superchunk decomposition reproduces the sequential recurrence.

Per chunk of L tokens (local index j), with the stabiliser m_prev at the
chunk start:
  b_j = sum_{l<=j} log sigmoid(f_l)      a_l = i_l - b_l
  M_j = max(m_prev, max_{l<=j} a_l)       m_j = b_j + M_j
  num_j = e^{m_prev-M_j} S~_prev^T q_j + sum_{l<=j} e^{a_l-M_j} (q_j.k_l) v_l
  den_j = e^{m_prev-M_j} n~_prev.q_j   + sum_{l<=j} e^{a_l-M_j} (q_j.k_l)
  h_j   = o_j num_j / max(|den_j + bias e^{-m_j}|, e^{-m_j})
  S~   <- e^{m_prev-M_L} S~_prev + sum_l e^{a_l-M_L} k_l v_l^T, m <- b_L + M_L
Chunks are grouped into superchunks of G chunks.  Pass 1 runs the state
update of every superchunk but the last from a zero state with m_prev = -inf,
giving (dS, dn, mu) and the superchunk's total log decay A.  Pass 2 scans
m_in' = max(A + m_in, mu), S_in' = e^{A+m_in-m_in'} S_in + e^{mu-m_in'} dS.
Pass 3 runs every superchunk from its S_in with readout and update.
Padded tokens past T carry log f = 0, i = -inf and zero q, k, v.
"""
import numpy as np


def _gates(fp, ip, valid):
    lf = np.where(valid, -np.logaddexp(0.0, -fp), 0.0)
    li = np.where(valid, ip, -np.inf)
    return lf, li


def _chunk(q, k, v, lf, li, o, bias, S, n, m_prev, nb, readout=True, normalise=True):
    """One chunk.  q,k [L,dqk]; v,o [L,dv]; S [nb,dqb,dvb]; n [dqk]."""
    L, dqk = q.shape
    dv = v.shape[1]
    dqb, dvb = dqk // nb, dv // nb
    b = np.cumsum(lf)
    a = li - b
    g = np.maximum.accumulate(a)
    M = np.maximum(m_prev, g)
    with np.errstate(invalid="ignore"):
        rs = np.exp(m_prev - M)                       # inter-chunk row scale
    rs = np.where(np.isfinite(M), rs, 0.0)
    W = np.exp(a[None, :] - M[:, None]) * np.tril(np.ones((L, L)))  # [j, l]
    W = np.nan_to_num(W)
    h = None
    if readout:
        num = np.zeros((L, dv))
        for be in range(nb):
            r, c = slice(be * dqb, (be + 1) * dqb), slice(be * dvb, (be + 1) * dvb)
            num[:, c] = rs[:, None] * (q[:, r] @ S[be]) + (W * (q[:, r] @ k[:, r].T)) @ v[:, c]
        mj = b + M
        if normalise:
            den = rs * (q @ n) + (W * (q @ k.T)).sum(axis=1) + bias * np.exp(-mj)
            h = o * num / np.maximum(np.abs(den), np.exp(-mj))[:, None]
        else:
            h = o * num
    alpha = np.exp(m_prev - M[-1]) if np.isfinite(m_prev) else 0.0
    w = np.exp(a - M[-1])
    S = S.copy()
    for be in range(nb):
        r, c = slice(be * dqb, (be + 1) * dqb), slice(be * dvb, (be + 1) * dvb)
        S[be] = alpha * S[be] + (k[:, r] * w[:, None]).T @ v[:, c]
    n = alpha * n + (w[:, None] * k).sum(axis=0)
    return h, S, n, b[-1] + M[-1]


def chunkwise(q, k, v, ip, fp, op=None, bias=None, C0=None, n0=None, m0=None,
              nb=1, L=64, G=4, normalise=True):
    """Same signature/outputs as ``oracle.mlstm_fwd`` (fp64 arrays)."""
    B, H, T, dqk = q.shape
    dv = v.shape[-1]
    dqb, dvb = dqk // nb, dv // nb
    NC = max(1, -(-T // L))
    NS = -(-NC // G)
    Tp = NC * L
    pad = lambda x, fill=0.0: np.concatenate(
        [x, np.full((Tp - T,) + x.shape[1:], fill)], axis=0)
    h = np.zeros((B, H, T, dv))
    Cf = np.zeros((B, H, nb, dqb, dvb))
    nf = np.zeros((B, H, dqk))
    mf = np.zeros((B, H))
    for bb in range(B):
        for hd in range(H):
            valid = np.arange(Tp) < T
            qq, kk, vv = pad(q[bb, hd]), pad(k[bb, hd]), pad(v[bb, hd])
            oo = np.ones((Tp, dv)) if op is None else 1.0 / (1.0 + np.exp(-pad(op[bb, hd])))
            lf, li = _gates(pad(fp[bb, hd]), pad(ip[bb, hd]), valid)
            bs = 0.0 if bias is None else bias[hd]
            sl = lambda c: slice(c * L, (c + 1) * L)
            # pass 1: local end state of every superchunk but the last
            dS, dn, mu, A = [], [], [], []
            for sc in range(NS - 1):
                S = np.zeros((nb, dqb, dvb))
                n = np.zeros(dqk)
                mloc = -np.inf
                for c in range(sc * G, (sc + 1) * G):
                    _, S, n, mloc = _chunk(qq[sl(c)], kk[sl(c)], vv[sl(c)], lf[sl(c)],
                                           li[sl(c)], None, bs, S, n, mloc, nb, readout=False)
                dS.append(S)
                dn.append(n)
                mu.append(mloc)
                A.append(lf[sc * G * L:(sc + 1) * G * L].sum())
            # pass 2: states at superchunk starts
            S = np.zeros((nb, dqb, dvb)) if C0 is None else C0[bb, hd].copy()
            n = np.zeros(dqk) if n0 is None else n0[bb, hd].copy()
            m = 0.0 if m0 is None else m0[bb, hd]
            Sin, nin, min_ = [S], [n], [m]
            for sc in range(NS - 1):
                mn = max(A[sc] + m, mu[sc])
                S = np.exp(A[sc] + m - mn) * S + np.exp(mu[sc] - mn) * dS[sc]
                n = np.exp(A[sc] + m - mn) * n + np.exp(mu[sc] - mn) * dn[sc]
                m = mn
                Sin.append(S)
                nin.append(n)
                min_.append(m)
            # pass 3: every superchunk from its start state
            hp = np.zeros((Tp, dv))
            for sc in range(NS):
                S, n, m = Sin[sc], nin[sc], min_[sc]
                for c in range(sc * G, min((sc + 1) * G, NC)):
                    hc, S, n, m = _chunk(qq[sl(c)], kk[sl(c)], vv[sl(c)], lf[sl(c)],
                                         li[sl(c)], oo[sl(c)], bs, S, n, m, nb,
                                         normalise=normalise)
                    hp[sl(c)] = hc
            h[bb, hd] = hp[:T]
            Cf[bb, hd], nf[bb, hd], mf[bb, hd] = S, n, m
    return h, Cf, nf, mf
