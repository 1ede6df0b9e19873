"""GPU parity of the chunkwise backward pass (mlstm_chunkwise_bwd through the C
ABI) against the oracle's step-by-step backward (oracle.mlstm_bwd) on the same
seeded inputs and incoming gradient.

Both recompute the forward from the inputs (the GPU in its own precision, the
oracle in fp64).  Metric as for the forward: per (batch, head)
slice, max |g - g_ref| / max |g_ref|, the largest over slices; 1e-4 for fp32,
2e-2 for bf16 inputs (the bias gradient: over heads).
"""
import numpy as np
import pytest
import torch

import oracle
from linear_recurrent_sequence_mlstm_amd import _lib as mlstm
from linear_recurrent_sequence_mlstm_amd.workloads import grad_output, mlstm_inputs, workload

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def slice_err(got, ref, lead=2):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    g = got.reshape(int(np.prod(got.shape[:lead])), -1)
    r = ref.reshape(g.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return float((np.abs(g - r).max(axis=1) / den).max())


def cpu(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def _state(B, H, dqk, dv, seed):
    g = torch.Generator().manual_seed(seed)
    C0 = torch.randn(B, H, 1, dqk, dv, generator=g) * 0.3
    n0 = torch.randn(B, H, dqk, generator=g) * 0.3
    m0 = torch.rand(B, H, generator=g) * 4 - 2
    return C0, n0, m0


def run_bwd(x, dev, seed, state=None):
    B, H, T, dqk = x.q.shape
    dv = x.v.shape[-1]
    dt = x.q.dtype
    dh = grad_output((B, H, T, dv), seed=seed, dtype="f32" if dt == torch.float32 else "bf16")
    g = x.to(dev)
    gs = None if state is None else tuple(t.to(dev) for t in state)
    out = mlstm.chunkwise_bwd(g.q, g.k, g.v, g.i_pre, g.f_pre, dh.to(dev), g.o_pre, g.bias, state=gs)
    torch.cuda.synchronize()
    st = (None, None, None) if state is None else (state[0].reshape(B, H, dqk, dv), state[1], state[2])
    ref = oracle.mlstm_bwd(x.q, x.k, x.v, x.i_pre, x.f_pre, dh, x.o_pre, x.bias, *st)
    return out, ref


def check(out, ref, tol, dbias_scale=None):
    """dbias_scale ([H], optional): judge the bias gradient, a sum over every
    token, against the magnitude of its terms rather than its own size."""
    errs = {}
    for name in ("dq", "dk", "dv", "di", "df", "do", "dC0", "dn0"):
        if out.get(name) is None:
            continue
        r = ref[name] if name != "dC0" else ref[name].reshape(out[name].shape)
        errs[name] = slice_err(cpu(out[name]), r)
    if out.get("dbias") is not None:
        if dbias_scale is None:
            errs["dbias"] = slice_err(cpu(out["dbias"]), ref["dbias"], lead=1)
        else:
            errs["dbias"] = float(np.abs(cpu(out["dbias"]) - ref["dbias"]).max() / np.max(dbias_scale))
    print({k: "%.2e" % v for k, v in errs.items()}, flush=True)
    bad = {k: v for k, v in errs.items() if not v < tol}
    assert not bad, bad


def test_bwd_cell_fp32_T60(gpu):
    x = workload("cell_fp32_T60")
    out, ref = run_bwd(x, gpu, seed=2001)
    check(out, ref, TOL[torch.float32])


def test_bwd_fp32_state_bias_ragged(gpu):
    x = mlstm_inputs(2, 2, 150, 64, 128, seed=2002, dtype="f32", k_scale=1 / 8, f_mix=True,
                     with_o=True, bias="uniform")
    out, ref = run_bwd(x, gpu, seed=2003, state=_state(2, 2, 64, 128, 2004))
    check(out, ref, TOL[torch.float32])


@pytest.mark.parametrize("dqk,dv,T,with_o,init", [(64, 128, 200, True, False), (128, 128, 256, False, True),
                                                  (64, 64, 1, True, True), (64, 192, 64, False, False)])
def test_bwd_bf16(gpu, dqk, dv, T, with_o, init):
    x = mlstm_inputs(2, 2, T, dqk, dv, seed=2100 + T + dqk, dtype="bf16", k_scale=dqk ** -0.5,
                     f_mix=True, with_o=with_o, bias="uniform")
    st = _state(2, 2, dqk, dv, 2200 + T) if init else None
    out, ref = run_bwd(x, gpu, seed=2300 + T, state=st)
    check(out, ref, TOL[torch.bfloat16])


def test_bwd_xlstm7b_head_shape(gpu):
    """The 7B layer's head shape (d_qk 256, d_v 512, k scaled by 1/16) over a
    ragged three-chunk sequence."""
    x = workload("xlstm7b_prefill_T8192", T=160, H=2)
    out, ref = run_bwd(x, gpu, seed=2005)
    check(out, ref, TOL[torch.bfloat16])


def test_bwd_xlstm7b_full_T8192_window(gpu):
    """The 7B prefill workload at full size (B=1, H=8, T=8192: the launch
    configuration bench.py times), dh non-zero on the last W = 320 tokens
    only.  Window tokens: every gradient against the oracle's backward over
    the window, started from the oracle's own state after the first T - W
    tokens.  Prefix tokens: dq is exactly zero, and the last prefix token's dk
    and dv follow from the window's initial-state gradient
    (dk = i' (dC0 v + dn0), dv = i' dC0^T k with i' = e^{i_pre - m}).

    The gradient jumps where |n.q + bias| crosses the floor 1 (the max in the
    denominator), and the GPU's states differ from fp64 by about 2e-3, so a
    token within that distance of the floor may take the other branch.  At
    tokens whose margin ||z| / floor - 1| (from the oracle, stepping through
    the window) is below 2e-2, dh is set to zero: there dh . h = 0, so dz~ = 0
    on both sides whichever branch each takes."""
    x = workload("xlstm7b_prefill_T8192")
    B, H, T, dqk = x.q.shape
    dv = x.v.shape[-1]
    W = 320
    cut = lambda t, a, b: t[:, :, a:b].contiguous()
    _, C, n, m = oracle.mlstm_fwd(*(cut(t, 0, T - W) for t in (x.q, x.k, x.v, x.i_pre, x.f_pre)))
    # margins to the denominator floor over the window
    Cs, ns, ms = C.copy(), n.copy(), m.copy()
    qn, kn, vn, ipn, fpn = (cpu(t) for t in (x.q, x.k, x.v, x.i_pre, x.f_pre))
    near = np.zeros((B, H, W), dtype=bool)
    for s in range(W):
        t = T - W + s
        oracle.mlstm_step(qn[:, :, t], kn[:, :, t], vn[:, :, t], ipn[:, :, t], fpn[:, :, t], Cs, ns, ms)
        z = np.einsum("bhd,bhd->bh", ns, qn[:, :, t])
        near[:, :, s] = np.abs(np.abs(z) * np.exp(ms) - 1) < 2e-2
    dh = grad_output((B, H, T, dv), seed=2006)
    dh[:, :, :T - W] = 0
    dh[:, :, T - W:][torch.from_numpy(near)] = 0
    print("window tokens near the floor (dh zeroed): %d of %d" % (int(near.sum()), near.size), flush=True)
    g = x.to(gpu)
    out = mlstm.chunkwise_bwd(g.q, g.k, g.v, g.i_pre, g.f_pre, dh.to(gpu))
    torch.cuda.synchronize()
    win = [cut(t, T - W, T) for t in (x.q, x.k, x.v, x.i_pre, x.f_pre)]
    ref = oracle.mlstm_bwd(*win, cut(dh, T - W, T), C0=C.reshape(B, H, dqk, dv), n0=n, m0=m)
    errs = {nm: slice_err(cpu(out[nm])[:, :, T - W:], ref[nm]) for nm in ("dq", "dk", "dv", "di", "df")}
    print({k: "%.2e" % v for k, v in errs.items()}, flush=True)
    assert all(v < TOL[torch.bfloat16] for v in errs.values()), errs
    assert float(out["dq"][:, :, :T - W].abs().max()) == 0.0
    t = T - W - 1
    iw = np.exp(ipn[:, :, t] - m)  # e^{i_pre - m} with m after token t
    dC0 = ref["dC0"]
    dk_ref = iw[..., None] * (np.einsum("bhdc,bhc->bhd", dC0, vn[:, :, t]) + ref["dn0"])
    dv_ref = iw[..., None] * np.einsum("bhdc,bhd->bhc", dC0, kn[:, :, t])
    e_k = slice_err(cpu(out["dk"])[:, :, t], dk_ref)
    e_v = slice_err(cpu(out["dv"])[:, :, t], dv_ref)
    print("last prefix token: dk %.2e dv %.2e" % (e_k, e_v), flush=True)
    assert e_k < TOL[torch.bfloat16] and e_v < TOL[torch.bfloat16], (e_k, e_v)


@pytest.mark.parametrize("G,dtype", [(2, "bf16"), (3, "bf16"), (3, "f32")])
def test_bwd_multichunk_superchunks(gpu, monkeypatch, G, dtype):
    """Superchunks of G chunks (the plan's override), so that the chunk-state
    walk steps through several chunks from each superchunk start state, with
    an initial state and a ragged tail."""
    monkeypatch.setenv("MLSTM_SUPERCHUNK_CHUNKS", str(G))
    x = mlstm_inputs(1, 2, 7 * 64 - 9, 64, 128, seed=2400 + G, dtype=dtype, k_scale=1 / 8, f_mix=True,
                     with_o=True, bias="uniform")
    out, ref = run_bwd(x, gpu, seed=2500 + G, state=_state(1, 2, 64, 128, 2600 + G))
    check(out, ref, TOL[x.q.dtype])


@pytest.mark.parametrize("dtype,B,H,T,dk,dv,with_state", [("f32", 1, 3, 150, 64, 64, True),
                                                          ("bf16", 2, 4, 200, 64, 128, False),
                                                          ("bf16", 1, 2, 300, 128, 128, True)])
def test_retention_bwd(gpu, dtype, B, H, T, dk, dv, with_state):
    from linear_recurrent_sequence_mlstm_amd.workloads import retention_inputs
    q, k, v = retention_inputs(B, H, T, dk, dv, seed=2700 + T, dtype=dtype)
    do = grad_output((B, H, T, dv), seed=2800 + T, dtype=dtype)
    S0 = torch.randn(B, H, dk, dv, generator=torch.Generator().manual_seed(2900)) * 0.3 if with_state else None
    out = mlstm.retention_chunkwise_bwd(q.to(gpu), k.to(gpu), v.to(gpu), do.to(gpu),
                                        S0=None if S0 is None else S0.to(gpu))
    torch.cuda.synchronize()
    ref = oracle.retention_bwd(q, k, v, do, None, S0)
    errs = {nm: slice_err(cpu(out[nm]), ref[nm]) for nm in ("dq", "dk", "dv", "dS0")}
    print(errs, flush=True)
    tol = TOL[q.dtype]
    assert all(e < tol for e in errs.values()), errs


def test_retention_bwd_msr_T2048_full(gpu):
    """The RetNet multi-scale retention workload at full size (B=8, H=4, d=64,
    T=2048, bf16), every gradient against the oracle."""
    q, k, v = workload("retnet_msr_T2048")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    do = grad_output((B, H, T, dv), seed=3001, scale=1 / 8)
    out = mlstm.retention_chunkwise_bwd(q.to(gpu), k.to(gpu), v.to(gpu), do.to(gpu))
    torch.cuda.synchronize()
    ref = oracle.retention_bwd(q, k, v, do)
    errs = {nm: slice_err(cpu(out[nm]), ref[nm]) for nm in ("dq", "dk", "dv", "dS0")}
    print(errs, flush=True)
    assert all(e < TOL[torch.bfloat16] for e in errs.values()), errs


@pytest.mark.parametrize("dtype,T,init,G", [("f32", 150, True, 0), ("bf16", 200, False, 0),
                                            ("bf16", 7 * 64 - 5, True, 3)])
def test_bwd_block_diagonal(gpu, monkeypatch, dtype, T, init, G):
    """Two memory blocks (d_qk = d_v = 64, 32 x 32 blocks) with the xLSTM-v2
    workload's distributions: k / 8, forget mixture, uniform bias; an initial
    block-diagonal state; superchunks of 3 chunks in the last case.

    The bias gradient is a sum over all tokens whose terms cancel (by about
    85x in the last case), so it is judged against the magnitude of its
    terms: the sum of |oracle dbias| over 16-token ranges of dh (dbias is
    linear in dh).  Every other gradient is judged as elsewhere."""
    if G:
        monkeypatch.setenv("MLSTM_SUPERCHUNK_CHUNKS", str(G))
    B, H, nb = 2, 2, 2
    x = mlstm_inputs(B, H, T, 64, 64, seed=3100 + T, dtype=dtype, nb=nb, k_scale=1 / 8, f_mix=True,
                     with_o=True, bias="uniform")
    dt = x.q.dtype
    dh = grad_output((B, H, T, 64), seed=3200 + T, dtype=dtype)
    st = None
    if init:
        g = torch.Generator().manual_seed(3300 + T)
        st = (torch.randn(B, H, nb, 32, 32, generator=g) * 0.3, torch.randn(B, H, 64, generator=g) * 0.3,
              torch.rand(B, H, generator=g) * 4 - 2)
    gx = x.to(gpu)
    out = mlstm.chunkwise_bwd(gx.q, gx.k, gx.v, gx.i_pre, gx.f_pre, dh.to(gpu), gx.o_pre, gx.bias,
                              state=None if st is None else tuple(t.to(gpu) for t in st), num_blocks=nb)
    torch.cuda.synchronize()
    args = (x.q, x.k, x.v, x.i_pre, x.f_pre)
    sargs = st if st is not None else (None, None, None)
    ref = oracle.mlstm_bwd(*args, dh, x.o_pre, x.bias, *sargs, num_blocks=nb)
    scale = np.zeros(H)
    for a in range(0, T, 16):
        part = torch.zeros_like(dh)
        part[:, :, a:a + 16] = dh[:, :, a:a + 16]
        scale += np.abs(oracle.mlstm_bwd(*args, part, x.o_pre, x.bias, *sargs, num_blocks=nb)["dbias"])
    check(out, ref, TOL[dt], dbias_scale=scale)


def near_floor(x, state, band=2e-2):
    """[B,H,T] mask of tokens whose |n.q + bias| lies within a relative band of
    the denominator floor 1 (by the oracle, stepping through the sequence):
    there the gradient jumps, and a bf16 run may take the other branch."""
    B, H, T, dqk = x.q.shape
    dv = x.v.shape[-1]
    q, k, v, ip, fp = (cpu(t) for t in (x.q, x.k, x.v, x.i_pre, x.f_pre))
    op = cpu(x.o_pre)
    bs = cpu(x.bias)
    if state is None:
        C, n, m = np.zeros((B, H, 1, dqk, dv)), np.zeros((B, H, dqk)), np.zeros((B, H))
    else:
        C, n, m = (t.double().numpy().copy() for t in state)
    mask = np.zeros((B, H, T), dtype=bool)
    for t in range(T):
        oracle.mlstm_step(q[:, :, t], k[:, :, t], v[:, :, t], ip[:, :, t], fp[:, :, t], C, n, m,
                          None if op is None else op[:, :, t], bs)
        z = np.einsum("bhd,bhd->bh", n, q[:, :, t]) * np.exp(m)
        if bs is not None:
            z = z + bs[None, :]
        mask[:, :, t] = np.abs(np.abs(z) - 1) < band
    return mask


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_long_sequence_two_level_scan(gpu, dtype):
    """257 chunks (T = 16421, ragged): the backward chunk scan runs in two
    levels (segments of 32 chunks, the last one a single chunk), with an
    initial state whose gradient comes out of the segment carries.  dh is
    zero at tokens within 2% of the denominator floor, as in the full 7B
    test (the gradient jumps there)."""
    B, H, T = 1, 2, 256 * 64 + 37
    x = mlstm_inputs(B, H, T, 64, 64, seed=3400, dtype=dtype, k_scale=1 / 8, f_mix=True, with_o=True,
                     bias="uniform")
    st = _state(B, H, 64, 64, 3402)
    mask = near_floor(x, st)
    dh = grad_output((B, H, T, 64), seed=3401, dtype=dtype)
    dh[torch.from_numpy(mask)] = 0
    print("tokens near the floor (dh zeroed): %d of %d" % (int(mask.sum()), mask.size), flush=True)
    g = x.to(gpu)
    out = mlstm.chunkwise_bwd(g.q, g.k, g.v, g.i_pre, g.f_pre, dh.to(gpu), g.o_pre, g.bias,
                              state=tuple(t.to(gpu) for t in st))
    torch.cuda.synchronize()
    ref = oracle.mlstm_bwd(x.q, x.k, x.v, x.i_pre, x.f_pre, dh, x.o_pre, x.bias, st[0].reshape(B, H, 64, 64),
                           st[1], st[2])
    check(out, ref, TOL[x.q.dtype])
