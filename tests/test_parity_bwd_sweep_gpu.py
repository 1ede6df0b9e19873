"""GPU parity of the chunkwise backward over a seeded sweep of small random
configurations: dtype, head shape, memory blocks, length, batch and heads,
superchunk size, and whether an initial state, an output gate and a gradient
arriving at the final state are given.  Every gradient is compared with the
oracle's step-by-step backward on the same inputs, with the bars of the other
backward tests: per (batch, head) slice 1e-4 for fp32 and 2e-2 for bf16, the
bias gradient against the same bar times the sum of its per-token terms
(the forward-error bound of a sum whose terms cancel), and dh set to zero at
tokens within 2 % of the denominator floor, where the gradient jumps.  A
second sweep does the same for the retention backward (head shape, length,
per-head or default decays, initial state, final-state gradient).
"""
import numpy as np
import pytest
import torch

import oracle
from linear_recurrent_sequence_mlstm_amd import _lib as mlstm
from linear_recurrent_sequence_mlstm_amd.workloads import grad_output, mlstm_inputs

from test_parity_bwd_gpu import TOL, check, cpu, near_floor, slice_err

pytestmark = pytest.mark.gpu

# (dtype, d_qk, num_blocks, admissible d_v)
SHAPES = [("f32", 64, 1, (64, 128)), ("bf16", 64, 1, (64, 128, 192)), ("bf16", 128, 1, (128, 256)),
          ("bf16", 256, 1, (128, 256, 512)), ("f32", 64, 2, (64,)), ("bf16", 64, 2, (64,))]


def _cases(n=18, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt, dqk, nb, dvs = SHAPES[i % len(SHAPES)]
        dv = int(rng.choice(dvs))
        out.append(dict(dt=dt, dqk=dqk, nb=nb, dv=dv, T=int(rng.integers(1, 260 if dqk * dv >= 65536 else 420)),
                        B=int(rng.integers(1, 3)), H=int(rng.integers(1, 3)), G=int(rng.choice([0, 0, 2, 3])),
                        init=bool(rng.random() < 0.5), with_o=bool(rng.random() < 0.5),
                        final=bool(rng.random() < 0.4), seed=8000 + 10 * i))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "%s_d%dx%d_nb%d_T%d_B%dH%d_G%d%s%s%s" % (
    c["dt"], c["dqk"], c["dv"], c["nb"], c["T"], c["B"], c["H"], c["G"], "_state" if c["init"] else "",
    "_o" if c["with_o"] else "", "_final" if c["final"] else ""))
def test_random_backward_configuration(gpu, monkeypatch, case):
    c = case
    if c["G"]:
        monkeypatch.setenv("MLSTM_SUPERCHUNK_CHUNKS", str(c["G"]))
    B, H, T, dqk, dv, nb, s = c["B"], c["H"], c["T"], c["dqk"], c["dv"], c["nb"], c["seed"]
    x = mlstm_inputs(B, H, T, dqk, dv, seed=s, dtype=c["dt"], nb=nb, k_scale=dqk ** -0.5, f_mix=True,
                     with_o=c["with_o"], bias="uniform")
    st = None
    if c["init"]:
        g = torch.Generator().manual_seed(s + 1)
        st = (torch.randn(B, H, nb, dqk // nb, dv // nb, generator=g) * 0.3,
              torch.randn(B, H, dqk, generator=g) * 0.3, torch.rand(B, H, generator=g) * 4 - 2)
    dh = grad_output((B, H, T, dv), seed=s + 2, dtype=c["dt"])
    # z = n.q + bias does not involve the memory: the walk to find the
    # near-floor tokens takes the full-head matrix form with a zero C0
    mask = near_floor(x, None if st is None else (torch.zeros(B, H, 1, dqk, dv), st[1], st[2]))
    dh[torch.from_numpy(mask)] = 0
    fin = None
    if c["final"]:
        g = torch.Generator().manual_seed(s + 3)
        fin = (torch.randn(B, H, nb, dqk // nb, dv // nb, generator=g), torch.randn(B, H, dqk, generator=g))
    gx = x.to(gpu)
    out = mlstm.chunkwise_bwd(gx.q, gx.k, gx.v, gx.i_pre, gx.f_pre, dh.to(gpu), gx.o_pre, gx.bias,
                              state=None if st is None else tuple(t.to(gpu) for t in st), num_blocks=nb,
                              final_grad=None if fin is None else tuple(t.to(gpu) for t in fin))
    torch.cuda.synchronize()
    sargs = st if st is not None else (None, None, None)
    ref = oracle.mlstm_bwd(x.q, x.k, x.v, x.i_pre, x.f_pre, dh, x.o_pre, x.bias, *sargs, num_blocks=nb,
                           dCT=None if fin is None else fin[0], dnT=None if fin is None else fin[1])
    tol = TOL[x.q.dtype]
    terms = np.abs(ref["dbias_t"]).sum(axis=(0, 2))
    e = float((np.abs(cpu(out["dbias"]) - ref["dbias"]) / np.maximum(terms, 1e-30)).max())
    print("near-floor tokens %d of %d; dbias %.2e of sum |dz_t|" % (int(mask.sum()), mask.size, e), flush=True)
    assert e < tol, e
    check(dict(out, dbias=None), ref, tol)


# retention backward: (dtype, d_k, admissible d_v)
RSHAPES = [("f32", 64, (64, 128)), ("bf16", 64, (64, 128, 256)), ("bf16", 128, (128, 256))]


def _rcases(n=9, seed=2027):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt, dk, dvs = RSHAPES[i % len(RSHAPES)]
        out.append(dict(dt=dt, dk=dk, dv=int(rng.choice(dvs)), T=int(rng.integers(1, 700)),
                        B=int(rng.integers(1, 3)), H=int(rng.integers(1, 5)), init=bool(rng.random() < 0.5),
                        gamma=bool(rng.random() < 0.4), final=bool(rng.random() < 0.4), seed=9000 + 10 * i))
    return out


@pytest.mark.parametrize("case", _rcases(), ids=lambda c: "%s_d%dx%d_T%d_B%dH%d%s%s%s" % (
    c["dt"], c["dk"], c["dv"], c["T"], c["B"], c["H"], "_state" if c["init"] else "",
    "_gamma" if c["gamma"] else "", "_final" if c["final"] else ""))
def test_random_retention_backward_configuration(gpu, case):
    from linear_recurrent_sequence_mlstm_amd.workloads import retention_inputs
    c = case
    B, H, T, dk, dv, s = c["B"], c["H"], c["T"], c["dk"], c["dv"], c["seed"]
    q, k, v = retention_inputs(B, H, T, dk, dv, seed=s, dtype=c["dt"])
    do = grad_output((B, H, T, dv), seed=s + 1, dtype=c["dt"])
    g = torch.Generator().manual_seed(s + 2)
    gamma = (1 - torch.rand(H, generator=g) * 0.1).float() if c["gamma"] else None
    S0 = torch.randn(B, H, dk, dv, generator=g) * 0.3 if c["init"] else None
    dST = torch.randn(B, H, dk, dv, generator=g) if c["final"] else None
    dev = torch.device(gpu)
    out = mlstm.retention_chunkwise_bwd(q.to(dev), k.to(dev), v.to(dev), do.to(dev),
                                        None if gamma is None else gamma.to(dev),
                                        None if S0 is None else S0.to(dev),
                                        dS_T=None if dST is None else dST.to(dev))
    torch.cuda.synchronize()
    ref = oracle.retention_bwd(q, k, v, do, gamma, S0, dS_T=dST)
    errs = {nm: slice_err(cpu(out[nm]), ref[nm]) for nm in ("dq", "dk", "dv", "dS0")}
    print(errs, flush=True)
    assert all(e < TOL[q.dtype] for e in errs.values()), errs
