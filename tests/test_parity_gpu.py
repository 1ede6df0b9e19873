"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle on
the same seeded inputs.

Error metric: for every (batch, head) slice, max |y - y_ref| / max |y_ref|
over all its elements; the test takes the largest over slices.  Bars: 1e-4
for the fp32 path, 2e-2 for bf16 inputs.  Final states are compared after
rescaling the stabilised state by e^{m_gpu - m_ref}; m itself to 1e-4
absolute.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_recurrent_sequence_mlstm_amd import _lib as mlstm
from linear_recurrent_sequence_mlstm_amd.workloads import mlstm_inputs, retention_inputs, workload

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


def check_state(gpu_state, ref, tol, m_tol=1e-4):
    C, n, m = (cpu(t) for t in gpu_state)
    Cr, nr, mr = ref
    assert np.max(np.abs(m - mr)) < m_tol
    sc = np.exp(m - mr)
    assert slice_err(C * sc[:, :, None, None, None], Cr) < tol
    assert slice_err(n * sc[:, :, None], nr) < tol


def run_both(x, dev, chunk=64, state=None, gpu_state=None):
    g = x.to(dev)
    h, st = mlstm.chunkwise_fwd(g.q, g.k, g.v, g.i_pre, g.f_pre, g.o_pre, g.bias, state=gpu_state,
                                num_blocks=x.num_blocks, chunk=chunk)
    torch.cuda.synchronize()
    ref = oracle.mlstm_fwd(x.q, x.k, x.v, x.i_pre, x.f_pre, x.o_pre, x.bias,
                           *(state if state is not None else (None, None, None)),
                           num_blocks=x.num_blocks)
    return h, st, ref


# ---------------------------------------------------------------- fp32 cell
@pytest.mark.parametrize("chunk", [64, 32, 16])
def test_cell_fp32_T60_chunkwise(gpu, chunk):
    x = workload("cell_fp32_T60")
    h, st, ref = run_both(x, gpu, chunk=chunk)
    assert slice_err(cpu(h), ref[0]) < TOL[torch.float32]
    check_state(st, ref[1:], TOL[torch.float32])


def test_cell_fp32_T60_step(gpu):
    x = workload("cell_fp32_T60")
    g = x.to(gpu)
    B, H, T, dqk = x.q.shape
    dv = x.v.shape[-1]
    C = torch.zeros(B, H, 1, dqk, dv, device=gpu)
    n = torch.zeros(B, H, dqk, device=gpu)
    m = torch.zeros(B, H, device=gpu)
    Cr, nr, mr = np.zeros((B, H, 1, dqk, dv)), np.zeros((B, H, dqk)), np.zeros((B, H))
    for t in range(T):
        h = mlstm.step(g.q[:, :, t].contiguous(), g.k[:, :, t].contiguous(), g.v[:, :, t].contiguous(),
                       g.i_pre[:, :, t].contiguous(), g.f_pre[:, :, t].contiguous(), C, n, m,
                       o_pre=g.o_pre[:, :, t].contiguous(), bias=g.bias)
        hr = oracle.mlstm_step(x.q[:, :, t], x.k[:, :, t], x.v[:, :, t], x.i_pre[:, :, t],
                               x.f_pre[:, :, t], Cr, nr, mr, o_pre=x.o_pre[:, :, t], bias=x.bias)
        assert slice_err(cpu(h), hr) < TOL[torch.float32], t
    check_state((C, n, m), (Cr, nr, mr), TOL[torch.float32])


# ------------------------------------------------------------ bf16 chunkwise
CASES = [
    # B, H, T, dqk, dv, nb, with_o, bias, f_mix
    (2, 2, 200, 64, 64, 1, True, "uniform", False),
    (2, 2, 1, 64, 64, 1, True, "uniform", False),
    (1, 2, 63, 64, 64, 1, False, None, False),
    (1, 2, 64, 64, 64, 1, False, None, False),
    (1, 2, 65, 64, 64, 1, False, None, True),
    (2, 2, 777, 64, 64, 2, False, "uniform", True),
    (1, 3, 1500, 64, 128, 2, True, "uniform", True),
    (1, 2, 300, 128, 256, 1, True, "uniform", False),
    (1, 2, 1000, 256, 512, 1, False, None, False),
    (1, 1, 333, 256, 512, 1, True, "uniform", True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dT%d_%dx%d_nb%d" % c[:6])
def test_chunkwise_bf16(gpu, case):
    B, H, T, dqk, dv, nb, with_o, bias, fmix = case
    x = mlstm_inputs(B, H, T, dqk, dv, seed=7 + T, dtype="bf16", nb=nb, k_scale=dqk ** -0.5,
                     f_mix=fmix, with_o=with_o, bias=bias)
    h, st, ref = run_both(x, gpu)
    assert slice_err(cpu(h), ref[0]) < TOL[torch.bfloat16]
    check_state(st, ref[1:], TOL[torch.bfloat16])


@pytest.mark.parametrize("dqk,dv,nb", [(64, 64, 1), (64, 64, 2), (256, 512, 1)])
def test_chunkwise_initial_state_and_split_run(gpu, dqk, dv, nb):
    """Run [0, T1) then [T1, T) carrying the state; both halves and the final
    state must match the oracle's single run (the state is the checkpoint)."""
    B, H, T, T1 = 1, 2, 900, 413
    x = mlstm_inputs(B, H, T, dqk, dv, seed=31, dtype="bf16", nb=nb, k_scale=dqk ** -0.5,
                     f_mix=True, with_o=True, bias="uniform")
    ref = oracle.mlstm_fwd(x.q, x.k, x.v, x.i_pre, x.f_pre, x.o_pre, x.bias, num_blocks=nb)
    g = x.to(gpu)
    sl = lambda t, s: t[:, :, s].contiguous()
    a, b = slice(0, T1), slice(T1, T)
    h1, st1 = mlstm.chunkwise_fwd(sl(g.q, a), sl(g.k, a), sl(g.v, a), sl(g.i_pre, a), sl(g.f_pre, a),
                                  sl(g.o_pre, a), g.bias, num_blocks=nb)
    h2, st2 = mlstm.chunkwise_fwd(sl(g.q, b), sl(g.k, b), sl(g.v, b), sl(g.i_pre, b), sl(g.f_pre, b),
                                  sl(g.o_pre, b), g.bias, state=st1, num_blocks=nb)
    torch.cuda.synchronize()
    assert slice_err(cpu(torch.cat([h1, h2], dim=2)), ref[0]) < TOL[torch.bfloat16]
    check_state(st2, ref[1:], TOL[torch.bfloat16])
    # in place: state_out aliasing the initial state
    st_alias = tuple(t.clone() for t in st1)
    h3, _ = mlstm.chunkwise_fwd(sl(g.q, b), sl(g.k, b), sl(g.v, b), sl(g.i_pre, b), sl(g.f_pre, b),
                                sl(g.o_pre, b), g.bias, state=st_alias, state_out=st_alias, num_blocks=nb)
    torch.cuda.synchronize()
    assert torch.equal(h3, h2)
    check_state(st_alias, ref[1:], TOL[torch.bfloat16])


@pytest.mark.parametrize("T", [1, 37, 64])
@pytest.mark.parametrize("dqk,dv,nb,dtype,with_o,norm_mode", [
    (256, 512, 1, "bf16", False, "vector"), (256, 512, 1, "bf16", True, "vector"),
    (256, 512, 1, "bf16", False, "scalar"), (64, 256, 1, "bf16", True, "vector"),
    (128, 256, 1, "bf16", False, "vector"), (64, 64, 2, "bf16", True, "vector"), (64, 128, 1, "f32", True, "vector")])
def test_short_call_single_launch(gpu, T, dqk, dv, nb, dtype, with_o, norm_mode):
    """A call of one chunk (one superchunk) runs as pass 3 alone, from the
    caller's initial state, forming the gate logs itself.  Against the oracle,
    and bit for bit against the three-launch plan, which an in-place call on
    a head wider than one work-group's d_v slice takes (its final n~ and m
    overwrite arrays the other slices still read)."""
    B, H = 2, 3
    x = mlstm_inputs(B, H, T, dqk, dv, seed=60 + T, dtype=dtype, nb=nb, k_scale=dqk ** -0.5, f_mix=True,
                     with_o=with_o, bias="uniform")
    rng = np.random.default_rng(61 + T)
    scalar = norm_mode == "scalar"
    C0 = rng.standard_normal((B, H, nb, dqk // nb, dv // nb)) * 0.3
    n0 = rng.standard_normal((B, H) if scalar else (B, H, dqk)) * 0.3
    m0 = rng.uniform(-2, 2, (B, H))
    ref = oracle.mlstm_fwd(x.q, x.k, x.v, x.i_pre, x.f_pre, x.o_pre, x.bias, C0, n0, m0, num_blocks=nb,
                           norm_mode=norm_mode)
    g = x.to(gpu)
    st0 = tuple(torch.tensor(a, dtype=torch.float32, device=gpu) for a in (C0, n0, m0))
    h1, st1 = mlstm.chunkwise_fwd(g.q, g.k, g.v, g.i_pre, g.f_pre, g.o_pre, g.bias, state=st0, num_blocks=nb,
                                  norm_mode=norm_mode)
    st_alias = tuple(t.clone() for t in st0)
    h2, _ = mlstm.chunkwise_fwd(g.q, g.k, g.v, g.i_pre, g.f_pre, g.o_pre, g.bias, state=st_alias,
                                state_out=st_alias, num_blocks=nb, norm_mode=norm_mode)
    torch.cuda.synchronize()
    tol = TOL[g.q.dtype]
    assert slice_err(cpu(h1), ref[0]) < tol
    C, n, m = (cpu(t) for t in st1)
    assert np.max(np.abs(m - ref[3])) < 1e-4
    sc = np.exp(m - ref[3])
    assert slice_err(C * sc[:, :, None, None, None], ref[1]) < tol
    assert slice_err(n * (sc if scalar else sc[:, :, None]), ref[2]) < tol
    assert torch.equal(h1, h2)
    for a, b in zip(st1, st_alias):
        assert torch.equal(a, b)


@pytest.mark.parametrize("chunk,T", [(16, 9), (16, 16), (32, 29), (32, 32)])
def test_short_call_single_launch_small_chunks(gpu, chunk, T):
    """Direct calls with fp32 chunks of 16 and 32 tokens (the gate wave's
    lanes repeat the chunk's tokens; the scans run per segment): against the
    oracle and bit for bit against the three-launch plan (in place, two d_v
    slices)."""
    B, H, dqk, dv = 2, 3, 64, 128
    x = mlstm_inputs(B, H, T, dqk, dv, seed=80 + T, dtype="f32", k_scale=1 / 8, f_mix=True, with_o=True,
                     bias="uniform")
    rng = np.random.default_rng(81 + T)
    C0, n0, m0 = rng.standard_normal((B, H, 1, dqk, dv)) * 0.3, rng.standard_normal((B, H, dqk)) * 0.3, \
        rng.uniform(-2, 2, (B, H))
    ref = oracle.mlstm_fwd(x.q, x.k, x.v, x.i_pre, x.f_pre, x.o_pre, x.bias, C0, n0, m0)
    g = x.to(gpu)
    st0 = tuple(torch.tensor(a, dtype=torch.float32, device=gpu) for a in (C0, n0, m0))
    h1, st1 = mlstm.chunkwise_fwd(g.q, g.k, g.v, g.i_pre, g.f_pre, g.o_pre, g.bias, state=st0, chunk=chunk)
    st_alias = tuple(t.clone() for t in st0)
    h2, _ = mlstm.chunkwise_fwd(g.q, g.k, g.v, g.i_pre, g.f_pre, g.o_pre, g.bias, state=st_alias,
                                state_out=st_alias, chunk=chunk)
    torch.cuda.synchronize()
    assert slice_err(cpu(h1), ref[0]) < TOL[torch.float32]
    check_state(st1, ref[1:], TOL[torch.float32])
    assert torch.equal(h1, h2)
    for a, b in zip(st1, st_alias):
        assert torch.equal(a, b)


def test_chunkwise_deterministic_and_writes_every_output(gpu):
    x = mlstm_inputs(1, 4, 1234, 256, 512, seed=5, dtype="bf16", k_scale=1 / 16).to(gpu)
    outs = []
    for _ in range(2):
        h = torch.full((1, 4, 1234, 512), float("nan"), dtype=torch.bfloat16, device=gpu)
        mlstm.chunkwise_fwd(x.q, x.k, x.v, x.i_pre, x.f_pre, h=h)
        outs.append(h)
    torch.cuda.synchronize()
    assert not torch.isnan(outs[0]).any()
    assert torch.equal(outs[0], outs[1])


# ------------------------------------------------- scalar normaliser reading
@pytest.mark.parametrize("case", [
    dict(B=1, H=2, T=300, dqk=256, dv=512, nb=1, dtype="bf16", f_mix=True, with_o=False, bias="uniform"),
    dict(B=2, H=2, T=200, dqk=64, dv=64, nb=2, dtype="bf16", f_mix=True, with_o=True, bias="uniform"),
    dict(B=1, H=3, T=100, dqk=64, dv=64, nb=1, dtype="f32", f_mix=False, with_o=True, bias="uniform"),
])
def test_chunkwise_scalar_normaliser(gpu, case):
    """norm_mode "scalar" (the XLSTMv2 page's printed n = f n + i): outputs
    and final (C, n, m) against the oracle's scalar mode, from an initial
    state carried over from a first run."""
    c = dict(case)
    dt = c.pop("dtype")
    x = mlstm_inputs(**c, dtype=dt, seed=41, k_scale=0.125)
    T1 = c["T"] // 3
    cut = lambda t, s: None if t is None else t[:, :, s].contiguous()
    xa = type(x)(*(cut(t, slice(0, T1)) for t in (x.q, x.k, x.v, x.i_pre, x.f_pre, x.o_pre)), x.bias,
                 x.num_blocks, x.chunk)
    xb = type(x)(*(cut(t, slice(T1, None)) for t in (x.q, x.k, x.v, x.i_pre, x.f_pre, x.o_pre)), x.bias,
                 x.num_blocks, x.chunk)
    ga, gb = xa.to(gpu), xb.to(gpu)
    ha, sta = mlstm.chunkwise_fwd(ga.q, ga.k, ga.v, ga.i_pre, ga.f_pre, ga.o_pre, ga.bias,
                                  num_blocks=x.num_blocks, norm_mode="scalar")
    assert tuple(sta[1].shape) == (x.q.shape[0], x.q.shape[1])
    hb, stb = mlstm.chunkwise_fwd(gb.q, gb.k, gb.v, gb.i_pre, gb.f_pre, gb.o_pre, gb.bias, state=sta,
                                  num_blocks=x.num_blocks, norm_mode="scalar")
    torch.cuda.synchronize()
    ref = oracle.mlstm_fwd(x.q, x.k, x.v, x.i_pre, x.f_pre, x.o_pre, x.bias, num_blocks=x.num_blocks,
                           norm_mode="scalar")
    tol = TOL[torch.bfloat16 if dt == "bf16" else torch.float32]
    assert slice_err(np.concatenate([cpu(ha), cpu(hb)], axis=2), ref[0]) < tol
    C, n, m = (cpu(t) for t in stb)
    Cr, nr, mr = ref[1:]
    assert np.max(np.abs(m - mr)) < 1e-4
    sc = np.exp(m - mr)
    assert slice_err(C * sc[:, :, None, None, None], Cr) < tol
    assert np.max(np.abs(n * sc - nr) / np.maximum(np.abs(nr), 1e-30)) < tol


def test_step_scalar_normaliser(gpu):
    """Decode steps in scalar mode after a scalar-mode prefill equal one
    oracle run over the whole sequence."""
    B, H, T, T1, dqk, dv = 2, 3, 90, 60, 64, 128
    x = mlstm_inputs(B, H, T, dqk, dv, dtype="bf16", seed=42, k_scale=0.125, with_o=True, bias="uniform")
    g = x.to(gpu)
    cut = lambda t: None if t is None else t[:, :, :T1].contiguous()
    _, (C, n, m) = mlstm.chunkwise_fwd(*(cut(t) for t in (g.q, g.k, g.v, g.i_pre, g.f_pre, g.o_pre)), g.bias,
                                       norm_mode="scalar")
    outs = []
    for t in range(T1, T):
        tok = lambda a: a[:, :, t].contiguous()
        outs.append(cpu(mlstm.step(tok(g.q), tok(g.k), tok(g.v), tok(g.i_pre), tok(g.f_pre), C, n, m,
                                   o_pre=tok(g.o_pre), bias=g.bias, norm_mode="scalar")))
    torch.cuda.synchronize()
    ref = oracle.mlstm_fwd(x.q, x.k, x.v, x.i_pre, x.f_pre, x.o_pre, x.bias, norm_mode="scalar")
    assert slice_err(np.stack(outs, axis=2), ref[0][:, :, T1:]) < TOL[torch.bfloat16]
    mm = cpu(m)
    assert np.max(np.abs(mm - ref[3])) < 1e-4
    nn_ = cpu(n) * np.exp(mm - ref[3])
    assert np.max(np.abs(nn_ - ref[2]) / np.abs(ref[2])) < TOL[torch.bfloat16]


# ------------------------------------------------ per-block normaliser reading
@pytest.mark.parametrize("B,H,T,dqk,dv,dtype", [(2, 2, 150, 64, 64, "bf16"), (1, 2, 130, 256, 512, "bf16"),
                                                 (1, 2, 70, 64, 64, "f32")])
def test_chunkwise_block_normaliser(gpu, B, H, T, dqk, dv, dtype):
    """norm_mode "block" with two memory blocks against the oracle's
    per-block mode (each block its own denominator), outputs and state."""
    x = mlstm_inputs(B, H, T, dqk, dv, dtype=dtype, seed=51, nb=2, k_scale=0.125, f_mix=True,
                     with_o=True, bias="uniform")
    g = x.to(gpu)
    h, st = mlstm.chunkwise_fwd(g.q, g.k, g.v, g.i_pre, g.f_pre, g.o_pre, g.bias, num_blocks=2,
                                norm_mode="block")
    torch.cuda.synchronize()
    assert tuple(st[1].shape) == (B, H, dqk)  # the per-block reading keeps the vector n
    ref = oracle.mlstm_fwd(x.q, x.k, x.v, x.i_pre, x.f_pre, x.o_pre, x.bias, num_blocks=2, norm_mode="block")
    tol = TOL[torch.bfloat16 if dtype == "bf16" else torch.float32]
    assert slice_err(cpu(h), ref[0]) < tol
    check_state(st, ref[1:], tol)


def test_step_block_normaliser(gpu):
    """Decode steps in per-block mode from a per-block prefill equal one
    oracle run."""
    B, H, T, T1, dqk, dv = 2, 2, 50, 30, 64, 128
    x = mlstm_inputs(B, H, T, dqk, dv, dtype="bf16", seed=52, nb=2, k_scale=0.125, bias="uniform")
    g = x.to(gpu)
    cut = lambda t: None if t is None else t[:, :, :T1].contiguous()
    _, (C, n, m) = mlstm.chunkwise_fwd(*(cut(t) for t in (g.q, g.k, g.v, g.i_pre, g.f_pre, g.o_pre)), g.bias,
                                       num_blocks=2, norm_mode="block")
    outs = []
    for t in range(T1, T):
        tok = lambda a: a[:, :, t].contiguous()
        outs.append(cpu(mlstm.step(tok(g.q), tok(g.k), tok(g.v), tok(g.i_pre), tok(g.f_pre), C, n, m,
                                   bias=g.bias, num_blocks=2, norm_mode="block")))
    torch.cuda.synchronize()
    ref = oracle.mlstm_fwd(x.q, x.k, x.v, x.i_pre, x.f_pre, x.o_pre, x.bias, num_blocks=2, norm_mode="block")
    assert slice_err(np.stack(outs, axis=2), ref[0][:, :, T1:]) < TOL[torch.bfloat16]
    check_state((C, n, m), ref[1:], TOL[torch.bfloat16])


# ------------------------------------------------------------ retention
@pytest.mark.parametrize("T,with_state", [(2048, False), (700, True), (50, False)])
def test_retention_bf16(gpu, T, with_state):
    B, H, d = 8 if T == 2048 else 2, 4, 64
    q, k, v = retention_inputs(B, H, T, d, d, seed=1002)
    S0 = torch.randn(B, H, d, d, generator=torch.Generator().manual_seed(3)) if with_state else None
    out, S = mlstm.retention_chunkwise_fwd(q.to(gpu), k.to(gpu), v.to(gpu),
                                           S0=None if S0 is None else S0.to(gpu))
    torch.cuda.synchronize()
    ref_out, ref_S = oracle.retention_fwd(q, k, v, S0=S0)
    assert slice_err(cpu(out), ref_out) < TOL[torch.bfloat16]
    assert slice_err(cpu(S), ref_S) < TOL[torch.bfloat16]


def test_retention_decay_matrix_form_full_size(gpu):
    """RetNet workload at full size against the page's parallel form
    ((Q K^T) * D) V evaluated in fp64 on the CPU."""
    q, k, v = workload("retnet_msr_T2048")
    out, _ = mlstm.retention_chunkwise_fwd(q.to(gpu), k.to(gpu), v.to(gpu), return_state=False)
    torch.cuda.synchronize()
    B, H, T, _ = q.shape
    t = torch.arange(T, dtype=torch.float64)
    diff = (t[:, None] - t[None, :])
    qd, kd, vd = q.double(), k.double(), v.double()
    errs = []
    for hd in range(H):
        g = 1.0 - 2.0 ** (-5 - hd)
        D = torch.where(diff >= 0, g ** diff.clamp(min=0), torch.zeros(()))
        ref = ((qd[:, hd] @ kd[:, hd].transpose(1, 2)) * D) @ vd[:, hd]
        errs.append(slice_err(cpu(out[:, hd]), ref.numpy(), lead=1))
    assert max(errs) < TOL[torch.bfloat16]


def test_retention_custom_gamma_fp32(gpu):
    B, H, T, d = 1, 2, 130, 64
    q, k, v = retention_inputs(B, H, T, d, d, seed=9, dtype="f32")
    gamma = torch.tensor([0.9, 0.5])
    out, S = mlstm.retention_chunkwise_fwd(q.to(gpu), k.to(gpu), v.to(gpu), gamma=gamma.to(gpu))
    torch.cuda.synchronize()
    ref_out, ref_S = oracle.retention_fwd(q, k, v, gamma=gamma)
    assert slice_err(cpu(out), ref_out) < TOL[torch.float32]
    assert slice_err(cpu(S), ref_S) < TOL[torch.float32]


@pytest.mark.parametrize("B,H,T,dk,dv,dtype,with_state,affine", [
    (8, 4, 2048, 64, 64, "bf16", False, True),   # the RetNet workload's shape
    (2, 3, 130, 64, 64, "bf16", True, False),    # ragged tail, initial state
    (1, 2, 100, 64, 64, "f32", True, True),
    (2, 2, 200, 128, 128, "bf16", False, True),
    # heads wider than one work-group: fp32 rows through the workspace, then
    # the row pass (d_v = 2 d_k, the value width RetNet uses; 4 slices)
    (2, 3, 333, 64, 128, "bf16", True, True),
    (1, 2, 150, 64, 256, "f32", False, True),
    (2, 2, 200, 128, 512, "bf16", True, False),
])
def test_retention_groupnorm(gpu, B, H, T, dk, dv, dtype, with_state, affine):
    """Retention with the per-head group norm against the oracle's retention
    followed by its group norm; the final state is unaffected by the norm."""
    q, k, v = retention_inputs(B, H, T, dk, dv, seed=31, dtype=dtype)
    g = torch.Generator().manual_seed(6)
    S0 = torch.randn(B, H, dk, dv, generator=g) * 0.1 if with_state else None
    w = torch.rand(H * dv, generator=g) + 0.5 if affine else None
    b = torch.randn(H * dv, generator=g) * 0.1 if affine else None
    gamma = torch.linspace(0.7, 0.99, H) if dtype == "f32" else None
    dv_ = lambda t: None if t is None else t.to(gpu)
    out, S = mlstm.retention_chunkwise_fwd(q.to(gpu), k.to(gpu), v.to(gpu), gamma=dv_(gamma), S0=dv_(S0),
                                           groupnorm=(dv_(w), dv_(b), 1e-5))
    torch.cuda.synchronize()
    ref_y, ref_S = oracle.retention_fwd(q, k, v, gamma=gamma, S0=S0)
    ref = oracle.groupnorm(ref_y, w, b, eps=1e-5)
    tol = TOL[torch.bfloat16 if dtype == "bf16" else torch.float32]
    assert slice_err(cpu(out), ref) < tol
    assert slice_err(cpu(S), ref_S) < tol


@pytest.mark.parametrize("B,H,dk,dv,dtype,custom_gamma", [
    (8, 4, 64, 64, "bf16", False), (2, 3, 128, 256, "f32", True), (3, 2, 256, 512, "bf16", True),
])
def test_retention_step(gpu, B, H, dk, dv, dtype, custom_gamma):
    """T decode steps from a random state, token by token through
    retention_step, against the oracle's retention recurrence over the same
    T tokens: every step's output and the final state."""
    T = 40
    q, k, v = retention_inputs(B, H, T, dk, dv, seed=21, dtype=dtype)
    S0 = torch.randn(B, H, dk, dv, generator=torch.Generator().manual_seed(5)) * 0.1
    gamma = torch.linspace(0.6, 0.99, H) if custom_gamma else None
    S = S0.to(gpu).contiguous()
    g = None if gamma is None else gamma.to(gpu)
    outs = []
    for t in range(T):
        o = mlstm.retention_step(q[:, :, t].contiguous().to(gpu), k[:, :, t].contiguous().to(gpu),
                                 v[:, :, t].contiguous().to(gpu), S, gamma=g)
        outs.append(cpu(o))
    torch.cuda.synchronize()
    ref_out, ref_S = oracle.retention_fwd(q, k, v, gamma=gamma, S0=S0)
    got = np.stack(outs, axis=2)
    tol = TOL[torch.bfloat16 if dtype == "bf16" else torch.float32]
    assert slice_err(got, ref_out) < tol
    assert slice_err(cpu(S), ref_S) < tol


def test_retention_step_matches_chunkwise(gpu):
    """Prefill by retention_chunkwise_fwd, then steps, equals one chunkwise
    call over the whole sequence (the state hand-over of the two paths)."""
    B, H, T, T1, d = 2, 4, 100, 70, 64
    q, k, v = (t.to(gpu) for t in retention_inputs(B, H, T, d, d, seed=8))
    out_all, S_all = mlstm.retention_chunkwise_fwd(q, k, v)
    _, S = mlstm.retention_chunkwise_fwd(q[:, :, :T1].contiguous(), k[:, :, :T1].contiguous(),
                                         v[:, :, :T1].contiguous())
    outs = [mlstm.retention_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(), S)
            for t in range(T1, T)]
    torch.cuda.synchronize()
    got = np.stack([cpu(o) for o in outs], axis=2)
    assert slice_err(got, cpu(out_all[:, :, T1:])) < TOL[torch.bfloat16]
    assert slice_err(cpu(S), cpu(S_all)) < TOL[torch.bfloat16]


# ------------------------------------------------------------ decode step
@pytest.mark.parametrize("B,H,dqk,dv,nb,with_o,bias", [
    (3, 2, 64, 64, 1, True, "uniform"), (2, 4, 64, 64, 2, False, "uniform"),
    (4, 2, 256, 512, 1, False, None), (2, 2, 128, 256, 2, True, "uniform"),
])
def test_step_bf16(gpu, B, H, dqk, dv, nb, with_o, bias):
    from linear_recurrent_sequence_mlstm_amd.workloads import decode_inputs
    S = 20
    x = decode_inputs(S, B, H, dqk, dv, seed=77, nb=nb, k_scale=dqk ** -0.5, with_o=with_o, bias=bias)
    g = x.to(gpu)
    C = torch.zeros(B, H, nb, dqk // nb, dv // nb, device=gpu)
    n = torch.zeros(B, H, dqk, device=gpu)
    m = torch.zeros(B, H, device=gpu)
    Cr, nr, mr = np.zeros((B, H, nb, dqk // nb, dv // nb)), np.zeros((B, H, dqk)), np.zeros((B, H))
    for s in range(S):
        h = mlstm.step(g.q[s], g.k[s], g.v[s], g.i_pre[s], g.f_pre[s], C, n, m,
                       o_pre=None if g.o_pre is None else g.o_pre[s], bias=g.bias, num_blocks=nb)
        hr = oracle.mlstm_step(x.q[s], x.k[s], x.v[s], x.i_pre[s], x.f_pre[s], Cr, nr, mr,
                               o_pre=None if x.o_pre is None else x.o_pre[s], bias=x.bias, num_blocks=nb)
        assert slice_err(cpu(h), hr) < TOL[torch.bfloat16], s
    check_state((C, n, m), (Cr, nr, mr), TOL[torch.bfloat16])


def test_step_matches_chunkwise(gpu):
    """Decode steps continuing a chunkwise prefill equal the oracle on the
    concatenated sequence (prefill state handed to the step kernel)."""
    B, H, T, dqk, dv = 1, 2, 150, 64, 64
    x = mlstm_inputs(B, H, T + 5, dqk, dv, seed=12, dtype="bf16", k_scale=1 / 8, bias="uniform")
    ref = oracle.mlstm_fwd(x.q, x.k, x.v, x.i_pre, x.f_pre, None, x.bias)
    g = x.to(gpu)
    sl = lambda t: t[:, :, :T].contiguous()
    h, (C, n, m) = mlstm.chunkwise_fwd(sl(g.q), sl(g.k), sl(g.v), sl(g.i_pre), sl(g.f_pre), bias=g.bias)
    C = C.clone()
    hs = []
    for t in range(T, T + 5):
        hs.append(mlstm.step(g.q[:, :, t].contiguous(), g.k[:, :, t].contiguous(), g.v[:, :, t].contiguous(),
                             g.i_pre[:, :, t].contiguous(), g.f_pre[:, :, t].contiguous(), C, n, m,
                             bias=g.bias).clone())
    torch.cuda.synchronize()
    full = torch.cat([h, torch.stack(hs, dim=2)], dim=2)
    assert slice_err(cpu(full), ref[0]) < TOL[torch.bfloat16]


def test_binding_rejects_bad_tensors(gpu):
    """The binding's one-expression check of the common case falls through
    to the specific errors: a tensor on the host, of another dtype, not
    contiguous or of the wrong shape is refused before anything reaches the
    library."""
    x = mlstm_inputs(1, 2, 16, 64, 64, seed=90, dtype="bf16", k_scale=1 / 8).to(gpu)
    good = dict(q=x.q, k=x.k, v=x.v, i_pre=x.i_pre, f_pre=x.f_pre)
    mlstm.chunkwise_fwd(**good)  # accepted
    torch.cuda.synchronize()
    bad = [
        (dict(good, k=x.k.cpu()), ValueError),                          # host tensor
        (dict(good, v=x.v.float()), TypeError),                         # dtype
        (dict(good, q=x.q.transpose(2, 3).contiguous().transpose(2, 3)), ValueError),  # not contiguous
        (dict(good, i_pre=x.i_pre[:, :, :8].contiguous()), ValueError),  # shape
    ]
    for kw, err in bad:
        with pytest.raises(err):
            mlstm.chunkwise_fwd(**kw)
