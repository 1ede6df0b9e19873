"""Pins of the oracle's backward pass (oracle.mlstm_bwd) against facts that do
not come from its code:
  * central finite differences of the oracle's forward (L = sum dh * h) for
    every input, initial state included, with the denominator floor active on
    some tokens and not on others;
  * torch autograd through an unstabilised fp64 recurrence written here from
    the cell's definition (C_t = f C + i k v^T, n_t = f n + i k,
    h = o * C^T q / max(|n.q + bias|, 1)), at lengths on both sides of the
    oracle's checkpoint segment.
"""
import numpy as np
import pytest
import torch

import oracle


def _case(seed, B, H, T, dqk, dv, with_o=True, bias=True, init=True, kscale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, dqk))
    k = rng.standard_normal((B, H, T, dqk)) / np.sqrt(dqk) * kscale
    v = rng.standard_normal((B, H, T, dv))
    ip = rng.standard_normal((B, H, T))
    fp = np.where(rng.random((B, H, T)) < 0.7, rng.normal(3, 1, (B, H, T)),
                  rng.normal(-2, 1, (B, H, T)))
    op = rng.standard_normal((B, H, T, dv)) if with_o else None
    bs = rng.uniform(-0.5, 0.5, H) if bias else None
    C0 = rng.standard_normal((B, H, dqk, dv)) * 0.3 if init else None
    n0 = rng.standard_normal((B, H, dqk)) * 0.3 if init else None
    m0 = rng.uniform(-2, 2, (B, H)) if init else None
    dh = rng.standard_normal((B, H, T, dv))
    return dict(q=q, k=k, v=v, i_pre=ip, f_pre=fp, o_pre=op, bias=bs, C0=C0, n0=n0, m0=m0), dh


def _fwd(a):
    B, H, T, dqk = a["q"].shape
    dv = a["v"].shape[-1]
    C0 = None if a["C0"] is None else a["C0"].reshape(B, H, 1, dqk, dv)
    return oracle.mlstm_fwd(a["q"], a["k"], a["v"], a["i_pre"], a["f_pre"], a["o_pre"],
                            a["bias"], C0, a["n0"], a["m0"])[0]


def _torch_h(t):
    """Unstabilised recurrence in true units, fp64, differentiable."""
    q, k, v, ip, fp = t["q"], t["k"], t["v"], t["i_pre"], t["f_pre"]
    B, H, T, dqk = q.shape
    dv = v.shape[-1]
    if t["C0"] is not None:
        C = t["C0"] * torch.exp(t["m0"])[..., None, None]
        n = t["n0"] * torch.exp(t["m0"])[..., None]
    else:
        C = torch.zeros(B, H, dqk, dv, dtype=torch.float64)
        n = torch.zeros(B, H, dqk, dtype=torch.float64)
    bias = t["bias"] if t["bias"] is not None else torch.zeros(H, dtype=torch.float64)
    hs, zs = [], []
    for s in range(T):
        f = torch.sigmoid(fp[:, :, s])[..., None]
        i = torch.exp(ip[:, :, s])[..., None]
        C = f[..., None] * C + (i * k[:, :, s])[..., :, None] * v[:, :, s][..., None, :]
        n = f * n + i * k[:, :, s]
        num = (C * q[:, :, s][..., :, None]).sum(-2)
        z = (n * q[:, :, s]).sum(-1) + bias
        den = torch.clamp(z.abs(), min=1.0)
        o = torch.sigmoid(t["o_pre"][:, :, s]) if t["o_pre"] is not None else 1.0
        hs.append(o * num / den[..., None])
        zs.append(z.detach())
    return torch.stack(hs, 2), torch.stack(zs, 2)


GRAD_OF = dict(q="dq", k="dk", v="dv", i_pre="di", f_pre="df", o_pre="do", bias="dbias",
               C0="dC0", n0="dn0")


def _relerr(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def test_bwd_pin_finite_differences():
    a, dh = _case(11, 1, 2, 9, 4, 3, kscale=3.0)
    # both sides of the denominator floor occur, none within reach of the kink
    _, z = _torch_h({n: (None if x is None else torch.from_numpy(x)) for n, x in a.items()})
    z = z.numpy()
    assert (np.abs(z) > 1).any() and (np.abs(z) < 1).any()
    assert np.min(np.abs(np.abs(z) - 1)) > 1e-3
    g = oracle.mlstm_bwd(dh=dh, **a)
    eps = 1e-6
    for name, gname in GRAD_OF.items():
        x = a[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = np.sum(dh * _fwd(a))
            x[idx] = keep - eps
            lm = np.sum(dh * _fwd(a))
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        err = _relerr(g[gname], fd)
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("T,with_o,bias,init", [(1, True, True, True), (17, False, True, False),
                                                (40, True, False, True), (64, True, True, False)])
def test_bwd_pin_torch_autograd(T, with_o, bias, init):
    a, dh = _case(100 + T, 2, 2, T, 8, 6, with_o=with_o, bias=bias, init=init, kscale=2.0)
    g = oracle.mlstm_bwd(dh=dh, **a)
    t = {n: (None if x is None else torch.tensor(x, requires_grad=True)) for n, x in a.items()}
    h, _ = _torch_h(t)
    h_or = _fwd(a)
    assert _relerr(h_or, h.detach().numpy()) < 1e-12
    (h * torch.from_numpy(dh)).sum().backward()
    for name, gname in GRAD_OF.items():
        if t[name] is None or name == "m0":
            continue
        err = _relerr(g[gname], t[name].grad.numpy())
        assert err < 1e-10, (name, T, err)
    if not init:  # gradient of a zero initial state is still returned
        C0 = torch.zeros(2, 2, 8, 6, dtype=torch.float64, requires_grad=True)
        n0 = torch.zeros(2, 2, 8, dtype=torch.float64, requires_grad=True)
        t2 = dict(t, C0=C0, n0=n0, m0=torch.zeros(2, 2, dtype=torch.float64))
        h2, _ = _torch_h(t2)
        (h2 * torch.from_numpy(dh)).sum().backward()
        assert _relerr(g["dC0"], C0.grad.numpy()) < 1e-10
        assert _relerr(g["dn0"], n0.grad.numpy()) < 1e-10


def test_retention_bwd_pin_finite_differences():
    rng = np.random.default_rng(21)
    B, H, T, dk, dv = 1, 2, 7, 3, 4
    a = dict(q=rng.standard_normal((B, H, T, dk)), k=rng.standard_normal((B, H, T, dk)),
             v=rng.standard_normal((B, H, T, dv)), S0=rng.standard_normal((B, H, dk, dv)))
    gamma = np.array([0.9, 0.7])
    do = rng.standard_normal((B, H, T, dv))
    g = oracle.retention_bwd(a["q"], a["k"], a["v"], do, gamma, a["S0"])
    eps = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("S0", "dS0")):
        x = a[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = np.sum(do * oracle.retention_fwd(a["q"], a["k"], a["v"], gamma, a["S0"])[0])
            x[idx] = keep - eps
            lm = np.sum(do * oracle.retention_fwd(a["q"], a["k"], a["v"], gamma, a["S0"])[0])
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        assert _relerr(g[gname], fd) < 1e-7, name


def test_retention_bwd_pin_parallel_form_autograd():
    """Autograd through the decay-matrix parallel form ((Q K^T) * D) V of the
    RetNet page ("Key Innovation: Retention Mechanism"), default gammas."""
    rng = np.random.default_rng(22)
    B, H, T, dk, dv = 2, 3, 40, 8, 6
    q, k, v, do = (rng.standard_normal(s) for s in ((B, H, T, dk), (B, H, T, dk), (B, H, T, dv), (B, H, T, dv)))
    g = oracle.retention_bwd(q, k, v, do)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    gam = torch.tensor([1 - 2.0 ** (-5 - h) for h in range(H)], dtype=torch.float64)
    n = torch.arange(T, dtype=torch.float64)
    expo = (n[:, None] - n[None, :])
    D = torch.where(expo >= 0, gam[:, None, None] ** expo.clamp(min=0), torch.zeros(()))
    out = ((tq @ tk.transpose(-1, -2)) * D) @ tv
    (out * torch.from_numpy(do)).sum().backward()
    for t, nm in ((tq, "dq"), (tk, "dk"), (tv, "dv")):
        assert _relerr(g[nm], t.grad.numpy()) < 1e-10, nm


def test_bwd_pin_finite_differences_block_diagonal():
    """Two memory blocks (the XLSTMv2 page's block-diagonal memory): the
    gradient of every input and of the block-diagonal initial state against
    central finite differences of the forward oracle with num_blocks=2."""
    a, dh = _case(31, 1, 2, 8, 4, 6, kscale=3.0)
    B, H, dqk, dv, nb = 1, 2, 4, 6, 2
    a["C0"] = np.random.default_rng(32).standard_normal((B, H, nb, dqk // nb, dv // nb)) * 0.3

    def fwd(a):
        return oracle.mlstm_fwd(a["q"], a["k"], a["v"], a["i_pre"], a["f_pre"], a["o_pre"], a["bias"],
                                a["C0"], a["n0"], a["m0"], num_blocks=nb)[0]

    g = oracle.mlstm_bwd(dh=dh, num_blocks=nb, **a)
    eps = 1e-6
    for name, gname in GRAD_OF.items():
        x = a[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = np.sum(dh * fwd(a))
            x[idx] = keep - eps
            lm = np.sum(dh * fwd(a))
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        assert _relerr(g[gname], fd) < 1e-6, name


def _fwd_state(a, nb=1):
    """h and the final stabilised state (C, n, m) of the forward oracle."""
    B, H, T, dqk = a["q"].shape
    dv = a["v"].shape[-1]
    C0 = None if a["C0"] is None else a["C0"].reshape(B, H, nb, dqk // nb, dv // nb)
    return oracle.mlstm_fwd(a["q"], a["k"], a["v"], a["i_pre"], a["f_pre"], a["o_pre"], a["bias"], C0,
                            a["n0"], a["m0"], num_blocks=nb)


def test_bwd_pin_final_state_gradient_finite_differences():
    """A gradient arriving at the final state: the loss
    L = sum dh * h + e^{m_T - m_ref} (<dC_T, S~_T> + <dn_T, n~_T>)
    is the loss on the true final state (C_T = S~_T e^{m_T}) scaled by the
    constant e^{-m_ref}, a smooth function of the inputs however the
    stabiliser moves; its central finite differences pin every gradient of
    oracle.mlstm_bwd(..., dCT, dnT)."""
    a, dh = _case(41, 1, 2, 9, 4, 3, kscale=3.0)
    rng = np.random.default_rng(42)
    B, H, dqk, dv = 1, 2, 4, 3
    dCT = rng.standard_normal((B, H, dqk, dv))
    dnT = rng.standard_normal((B, H, dqk))
    _, _, _, m_ref = _fwd_state(a)
    m_ref = m_ref.copy()

    def loss(a):
        h, C, n, m = _fwd_state(a)
        s = np.exp(m - m_ref)
        return (np.sum(dh * h) + np.sum(s[..., None, None] * dCT * C.reshape(B, H, dqk, dv))
                + np.sum(s[..., None] * dnT * n))

    g = oracle.mlstm_bwd(dh=dh, dCT=dCT, dnT=dnT, **a)
    g0 = oracle.mlstm_bwd(dh=dh, **a)
    assert _relerr(g["dk"], g0["dk"]) > 1e-3  # the final-state term is not negligible here
    eps = 1e-6
    for name, gname in GRAD_OF.items():
        x = a[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = loss(a)
            x[idx] = keep - eps
            lm = loss(a)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        assert _relerr(g[gname], fd) < 1e-6, name


@pytest.mark.parametrize("T,init", [(1, True), (23, False), (50, True)])
def test_bwd_pin_final_state_gradient_autograd(T, init):
    """The same loss through torch autograd on the unstabilised recurrence of
    this file: the final-state term is <dC_T e^{-m_T}, C_T> + <dn_T e^{-m_T}, n_T>
    in true units (m_T from the forward oracle, a constant)."""
    a, dh = _case(200 + T, 2, 2, T, 8, 6, init=init, kscale=2.0)
    rng = np.random.default_rng(300 + T)
    dCT = rng.standard_normal((2, 2, 8, 6))
    dnT = rng.standard_normal((2, 2, 8))
    g = oracle.mlstm_bwd(dh=dh, dCT=dCT, dnT=dnT, **a)
    _, _, _, mT = _fwd_state(a)
    t = {n: (None if x is None else torch.tensor(x, requires_grad=True)) for n, x in a.items()}
    h, _, CT, nT = _torch_h_state(t)
    s = torch.from_numpy(np.exp(-mT))
    L = ((h * torch.from_numpy(dh)).sum() + (s[..., None, None] * torch.from_numpy(dCT) * CT).sum()
         + (s[..., None] * torch.from_numpy(dnT) * nT).sum())
    L.backward()
    for name, gname in GRAD_OF.items():
        if t[name] is None or name == "m0":
            continue
        assert _relerr(g[gname], t[name].grad.numpy()) < 1e-10, (name, T)


def _torch_h_state(t):
    """_torch_h that also returns the final true state (C_T, n_T)."""
    q, k, v, ip, fp = t["q"], t["k"], t["v"], t["i_pre"], t["f_pre"]
    B, H, T, dqk = q.shape
    dv = v.shape[-1]
    if t["C0"] is not None:
        C = t["C0"] * torch.exp(t["m0"])[..., None, None]
        n = t["n0"] * torch.exp(t["m0"])[..., None]
    else:
        C = torch.zeros(B, H, dqk, dv, dtype=torch.float64)
        n = torch.zeros(B, H, dqk, dtype=torch.float64)
    bias = t["bias"] if t["bias"] is not None else torch.zeros(H, dtype=torch.float64)
    hs = []
    for s in range(T):
        f = torch.sigmoid(fp[:, :, s])[..., None]
        i = torch.exp(ip[:, :, s])[..., None]
        C = f[..., None] * C + (i * k[:, :, s])[..., :, None] * v[:, :, s][..., None, :]
        n = f * n + i * k[:, :, s]
        num = (C * q[:, :, s][..., :, None]).sum(-2)
        z = (n * q[:, :, s]).sum(-1) + bias
        den = torch.clamp(z.abs(), min=1.0)
        o = torch.sigmoid(t["o_pre"][:, :, s]) if t["o_pre"] is not None else 1.0
        hs.append(o * num / den[..., None])
    return torch.stack(hs, 2), None, C, n


def test_bwd_pin_split_chaining():
    """Backward of a split run: the second part's initial-state gradients,
    passed as the first part's final-state gradients, give the gradients of
    the whole run (the state carry of the forward, run backwards)."""
    a, dh = _case(51, 2, 2, 30, 6, 5, kscale=2.0)
    T1 = 13
    full = oracle.mlstm_bwd(dh=dh, **a)
    part = lambda x, lo, hi: None if x is None else x[:, :, lo:hi]
    seq = ("q", "k", "v", "i_pre", "f_pre", "o_pre")
    a1 = dict(a, **{n: part(a[n], 0, T1) for n in seq})
    _, C1, n1, m1 = _fwd_state(a1)
    a2 = dict(a, **{n: part(a[n], T1, 30) for n in seq}, C0=C1.reshape(2, 2, 6, 5), n0=n1, m0=m1)
    g2 = oracle.mlstm_bwd(dh=dh[:, :, T1:], **a2)
    g1 = oracle.mlstm_bwd(dh=dh[:, :, :T1], dCT=g2["dC0"], dnT=g2["dn0"], **a1)
    for nm in ("dq", "dk", "dv", "di", "df", "do"):
        got = np.concatenate([g1[nm], g2[nm]], axis=2)
        assert _relerr(got, full[nm]) < 1e-11, nm
    assert _relerr(g1["dbias"] + g2["dbias"], full["dbias"]) < 1e-11
    assert _relerr(g1["dC0"], full["dC0"]) < 1e-11 and _relerr(g1["dn0"], full["dn0"]) < 1e-11


def test_bwd_pin_bias_terms():
    """The per-token terms of the bias gradient: where |z_t| > 1 (z_t = n_t . q_t
    + bias in true units), h_t = o * num / |z_t|, so d(dh_t . h_t)/d bias =
    -(dh_t . h_t) sign(z_t) / |z_t|, else 0; h and z from the unstabilised
    recurrence of this file.  Their sum over the batch and tokens is dbias,
    and the oracle's reported z is that recurrence's z."""
    a, dh = _case(61, 2, 3, 40, 8, 6, kscale=3.0)
    g = oracle.mlstm_bwd(dh=dh, **a)
    t = {n: (None if x is None else torch.from_numpy(x)) for n, x in a.items()}
    h, z = _torch_h(t)
    h, z = h.numpy(), z.numpy()
    assert (np.abs(z) > 1).any() and (np.abs(z) < 1).any()
    ref = np.where(np.abs(z) > 1, -np.sum(dh * h, axis=-1) * np.sign(z) / np.abs(z), 0.0)
    assert _relerr(g["dbias_t"], ref) < 1e-10
    assert _relerr(g["dbias_t"].sum(axis=(0, 2)), g["dbias"]) < 1e-12
    assert _relerr(g["z"], z) < 1e-12


def test_retention_bwd_pin_final_state_finite_differences():
    """Retention with a gradient arriving at the final state: central finite
    differences of sum(dout * out) + <dS_T, S_T> (S_T from the forward)."""
    rng = np.random.default_rng(23)
    B, H, T, dk, dv = 1, 2, 7, 3, 4
    a = dict(q=rng.standard_normal((B, H, T, dk)), k=rng.standard_normal((B, H, T, dk)),
             v=rng.standard_normal((B, H, T, dv)), S0=rng.standard_normal((B, H, dk, dv)))
    gamma = np.array([0.9, 0.7])
    do = rng.standard_normal((B, H, T, dv))
    dST = rng.standard_normal((B, H, dk, dv))

    def loss():
        out, S = oracle.retention_fwd(a["q"], a["k"], a["v"], gamma, a["S0"])
        return np.sum(do * out) + np.sum(dST * S)

    g = oracle.retention_bwd(a["q"], a["k"], a["v"], do, gamma, a["S0"], dS_T=dST)
    eps = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("S0", "dS0")):
        x = a[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = loss()
            x[idx] = keep - eps
            lm = loss()
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        assert _relerr(g[gname], fd) < 1e-7, name
