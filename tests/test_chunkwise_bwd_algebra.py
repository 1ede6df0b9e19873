"""The chunkwise backward algebra in plain numpy fp64, checked against the
oracle's step-by-step backward before (and independently of) any GPU code.

Per chunk of L tokens with local index j, in-chunk forget sums b_j, a_j =
li_j - b_j, M_j = max(m_prev, max_{l<=j} a_l) and chunk-end M_L (the forward's
stabiliser), the gradients of sum(dh * h) are
  dn~_j = o_j dh_j / den~_j,  dz~_j = -(dh_j . h_j) sign(z~_j) / den~_j if
          |z~_j| > e^{-m_j} else 0,
  E_jl = e^{a_l - M_j} (l <= j),  D'_jl = E_jl (dn~_j . v_l + dz~_j),
  dq_j = sum_l D'_jl k_l + e^{m_prev - M_j} (S~_prev dn~_j + n~_prev dz~_j),
  dk_j = sum_l D'_lj q_l + w_j (G_end v_j + g_end),   w_j = e^{a_j - M_L},
  dv_j = sum_l E_lj (q_l . k_j) dn~_l + w_j G_end^T k_j,
with the backward state at the end of each chunk from a reverse scan
  G_end(c-1) = e^{m_prev - M_L} G_end(c) + sum_j e^{m_prev - M_j} q_j dn~_j^T
(and its normaliser column with dz~_j), d i_pre_j = k_j . dk_j, d log f from
the reverse cumulative sum of q_t . dq_t - k_t . dk_t over the sequence, and
the initial-state gradient G_end(-1).  q_t, k_t enter h only as e^{F_t} q_t
and e^{i_t - F_t} k_t (F the cumulative log forget gate), hence the last two
identities.
"""
import numpy as np
import pytest

import oracle


def _sig(x):
    return 1 / (1 + np.exp(-x))


def chunkwise_bwd(q, k, v, ip, fp, op, bs, C0, n0, m0, dh, L):
    B, H, T, dqk = q.shape
    dv = v.shape[-1]
    NC = (T + L - 1) // L
    out = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v))}
    out["di"] = np.zeros((B, H, T))
    out["df"] = np.zeros((B, H, T))
    out["do"] = np.zeros_like(v) if op is not None else None
    out["dbias"] = np.zeros(H)
    out["dC0"] = np.zeros((B, H, dqk, dv))
    out["dn0"] = np.zeros((B, H, dqk))
    for b in range(B):
        for hd in range(H):
            bias = bs[hd] if bs is not None else 0.0
            lf = -np.logaddexp(0, -fp[b, hd])
            li = ip[b, hd]
            S = C0[b, hd].copy() if C0 is not None else np.zeros((dqk, dv))
            n = n0[b, hd].copy() if n0 is not None else np.zeros(dqk)
            m = m0[b, hd] if m0 is not None else 0.0
            # forward: chunk start states and stabiliser quantities
            st = []
            for c in range(NC):
                t0, t1 = c * L, min(T, c * L + L)
                bcs = np.cumsum(lf[t0:t1])
                a = li[t0:t1] - bcs
                M = np.maximum(m, np.maximum.accumulate(a))
                st.append((S.copy(), n.copy(), m, bcs, a, M))
                w = np.exp(a - M[-1])
                dec = np.exp(m - M[-1])
                S = dec * S + (w[:, None] * k[b, hd, t0:t1]).T @ v[b, hd, t0:t1]
                n = dec * n + w @ k[b, hd, t0:t1]
                m = bcs[-1] + M[-1]
            # per chunk: readout recomputed, dn~, dz~, D', dq and the local
            # backward-state contribution U
            per = []
            for c in range(NC):
                t0, t1 = c * L, min(T, c * L + L)
                Sp, npv, mp, bcs, a, M = st[c]
                Q, K, V = q[b, hd, t0:t1], k[b, hd, t0:t1], v[b, hd, t0:t1]
                Lc = t1 - t0
                E = np.tril(np.exp(a[None, :] - M[:, None]))
                P = E * (Q @ K.T)
                al = np.exp(mp - M)
                em = np.exp(-(bcs + M))
                num = P @ V + al[:, None] * (Q @ Sp)
                z = P.sum(1) + al * (Q @ npv) + bias * em
                den = np.maximum(np.abs(z), em)
                o = _sig(op[b, hd, t0:t1]) if op is not None else np.ones((Lc, dv))
                h = o * num / den[:, None]
                dN = o * dh[b, hd, t0:t1] / den[:, None]
                s = np.sum(dh[b, hd, t0:t1] * h, 1)
                dz = np.where(np.abs(z) > em, -s * np.sign(z) / den, 0.0)
                if op is not None:
                    out["do"][b, hd, t0:t1] = dh[b, hd, t0:t1] * h * (1 - o)
                out["dbias"][hd] += np.sum(em * dz)
                Dp = E * (dN @ V.T + dz[:, None])
                out["dq"][b, hd, t0:t1] = Dp @ K + al[:, None] * (dN @ Sp.T + dz[:, None] * npv[None, :])
                U = (al[:, None] * Q).T @ dN
                u = (al * dz) @ Q
                per.append((Dp, P, dN, U, u, np.exp(a - M[-1]), np.exp(mp - M[-1])))
            # reverse scan of the backward state over chunks
            G = np.zeros((dqk, dv))
            g = np.zeros(dqk)
            for c in range(NC - 1, -1, -1):
                t0, t1 = c * L, min(T, c * L + L)
                Dp, P, dN, U, u, w, dec = per[c]
                Q, K, V = q[b, hd, t0:t1], k[b, hd, t0:t1], v[b, hd, t0:t1]
                out["dk"][b, hd, t0:t1] = Dp.T @ Q + w[:, None] * (V @ G.T + g[None, :])
                out["dv"][b, hd, t0:t1] = P.T @ dN + w[:, None] * (K @ G)
                G = dec * G + U
                g = dec * g + u
            out["dC0"][b, hd] = G
            out["dn0"][b, hd] = g
            kdk = np.sum(k[b, hd] * out["dk"][b, hd], 1)
            qdq = np.sum(q[b, hd] * out["dq"][b, hd], 1)
            out["di"][b, hd] = kdk
            dlf = np.cumsum((qdq - kdk)[::-1])[::-1]
            out["df"][b, hd] = dlf * _sig(-fp[b, hd])
    return out


@pytest.mark.parametrize("T,L,init,with_o", [(1, 4, False, True), (30, 8, True, True),
                                             (64, 16, False, False), (61, 16, True, True)])
def test_chunkwise_bwd_algebra_equals_oracle(T, L, init, with_o):
    rng = np.random.default_rng(7 + T)
    B, H, dqk, dv = 2, 2, 8, 6
    q = rng.standard_normal((B, H, T, dqk))
    k = rng.standard_normal((B, H, T, dqk)) / np.sqrt(dqk) * 2
    v = rng.standard_normal((B, H, T, dv))
    ip = rng.standard_normal((B, H, T)) * 2
    fp = np.where(rng.random((B, H, T)) < 0.7, rng.normal(3, 1, (B, H, T)),
                  rng.normal(-2, 1, (B, H, T)))
    op = rng.standard_normal((B, H, T, dv)) if with_o else None
    bs = rng.uniform(-0.5, 0.5, H)
    C0 = rng.standard_normal((B, H, dqk, dv)) * 0.3 if init else None
    n0 = rng.standard_normal((B, H, dqk)) * 0.3 if init else None
    m0 = rng.uniform(-2, 2, (B, H)) if init else None
    dh = rng.standard_normal((B, H, T, dv))
    ref = oracle.mlstm_bwd(q, k, v, ip, fp, dh, op, bs, C0, n0, m0)
    got = chunkwise_bwd(q, k, v, ip, fp, op, bs, C0, n0, m0, dh, L)
    for name in ("dq", "dk", "dv", "di", "df", "do", "dbias", "dC0", "dn0"):
        if ref[name] is None:
            continue
        # (a floor for gradients that vanish exactly, e.g. df at T = 1 from a
        # zero state, where the identity's two terms cancel up to rounding)
        err = np.max(np.abs(got[name] - ref[name])) / max(np.max(np.abs(ref[name])), 1e-3)
        assert err < 1e-11, (name, err)
