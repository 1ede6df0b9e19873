"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (default chunk and superchunk plan, caller-provided outputs
and workspace), against the fp64 oracle on the same seeded inputs.

Error metric and bars as in test_parity_gpu: per (batch, head) slice,
max |y - y_ref| / max |y_ref|; 2e-2 for bf16 inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_recurrent_sequence_mlstm_amd import _lib as mlstm
from linear_recurrent_sequence_mlstm_amd.workloads import workload

from test_parity_gpu import TOL, check_state, cpu, slice_err

pytestmark = pytest.mark.gpu


def _chunkwise_like_bench(g, dev):
    B, H, T, dqk = g.q.shape
    dv = g.v.shape[-1]
    nb = g.num_blocks
    h = torch.empty(B, H, T, dv, dtype=g.q.dtype, device=dev)
    st = (torch.empty(B, H, nb, dqk // nb, dv // nb, device=dev), torch.empty(B, H, dqk, device=dev),
          torch.empty(B, H, device=dev))
    ws = torch.empty(mlstm.chunkwise_workspace_bytes(B, H, T, dqk, dv, nb, dtype=g.q.dtype),
                     dtype=torch.uint8, device=dev)
    mlstm.chunkwise_fwd(g.q, g.k, g.v, g.i_pre, g.f_pre, g.o_pre, g.bias, num_blocks=nb, h=h,
                        state_out=st, workspace=ws)
    torch.cuda.synchronize()
    return h, st


def test_xlstm7b_prefill_full_size(gpu):
    """B=1, 8 heads, d_qk=256, d_v=512, T=8192: every output and the final state."""
    x = workload("xlstm7b_prefill_T8192")
    h, st = _chunkwise_like_bench(x.to(gpu), gpu)
    ref = oracle.mlstm_fwd(x.q, x.k, x.v, x.i_pre, x.f_pre, x.o_pre, x.bias, num_blocks=x.num_blocks)
    assert slice_err(cpu(h), ref[0]) < TOL[torch.bfloat16]
    check_state(st, ref[1:], TOL[torch.bfloat16])


def test_xlstm2_blockdiag_T65536_full_size(gpu):
    """B=4, 4 heads, d=64 in two 32x32 blocks, T=65536, biased normaliser,
    bimodal forget gates: every output and the final state."""
    x = workload("xlstm2_blockdiag_T65536")
    h, st = _chunkwise_like_bench(x.to(gpu), gpu)
    ref = oracle.mlstm_fwd(x.q, x.k, x.v, x.i_pre, x.f_pre, x.o_pre, x.bias, num_blocks=x.num_blocks)
    assert slice_err(cpu(h), ref[0]) < TOL[torch.bfloat16]
    check_state(st, ref[1:], TOL[torch.bfloat16])


def test_xlstm7b_decode_128_steps_sampled(gpu):
    """B=256, 8 heads, 1 GiB fp32 state updated in place over 128 steps, as
    the benchmark runs it.  The oracle follows 32 sampled (batch, head)
    sequences (corners included): their h at every step and final state."""
    d = workload("xlstm7b_decode_B256")
    S, B, H, dqk = d.q.shape
    dv = d.v.shape[-1]
    g = d.to(gpu)
    C = torch.zeros(B, H, 1, dqk, dv, device=gpu)
    n = torch.zeros(B, H, dqk, device=gpu)
    m = torch.zeros(B, H, device=gpu)
    h = torch.empty(B, H, dv, dtype=torch.bfloat16, device=gpu)
    rng = np.random.default_rng(4)
    pairs = [(0, 0), (B - 1, H - 1), (B // 2, 3)] + [(int(b), int(hh)) for b, hh in
                                                      zip(rng.integers(0, B, 29), rng.integers(0, H, 29))]
    bi = torch.tensor([p[0] for p in pairs])
    hi = torch.tensor([p[1] for p in pairs])
    hs = []
    for s in range(S):
        mlstm.step(g.q[s], g.k[s], g.v[s], g.i_pre[s], g.f_pre[s], C, n, m, bias=g.bias, h=h)
        hs.append(h[bi.to(gpu), hi.to(gpu)].clone())
    torch.cuda.synchronize()
    got = torch.stack(hs, dim=1)[None]  # [1, P, S, dv]
    # sampled sequences as P heads of one batch: [1, P, S, d]
    sel = lambda t: t[:, bi, hi].permute(1, 0, 2)[None].contiguous()
    sel_g = lambda t: t[:, bi, hi].permute(1, 0)[None].contiguous()
    bias = None if d.bias is None else d.bias[hi].contiguous()
    ref = oracle.mlstm_fwd(sel(d.q), sel(d.k), sel(d.v), sel_g(d.i_pre), sel_g(d.f_pre), None, bias)
    assert slice_err(cpu(got), ref[0]) < TOL[torch.bfloat16]
    st = (C[bi.to(gpu), hi.to(gpu)][None], n[bi.to(gpu), hi.to(gpu)][None], m[bi.to(gpu), hi.to(gpu)][None])
    check_state(st, ref[1:], TOL[torch.bfloat16])


def test_xlstm7b_decode_all_sequences_first_8_steps(gpu):
    """The same decode workload on every one of its 2048 (batch, head)
    sequences: h at each of the first 8 steps and the whole 1 GiB state after
    them, against the oracle run on all sequences."""
    d = workload("xlstm7b_decode_B256")
    S8 = 8
    _, B, H, dqk = d.q.shape
    dv = d.v.shape[-1]
    g = d.to(gpu)
    C = torch.zeros(B, H, 1, dqk, dv, device=gpu)
    n = torch.zeros(B, H, dqk, device=gpu)
    m = torch.zeros(B, H, device=gpu)
    hs = []
    for s in range(S8):
        h = torch.empty(B, H, dv, dtype=torch.bfloat16, device=gpu)
        mlstm.step(g.q[s], g.k[s], g.v[s], g.i_pre[s], g.f_pre[s], C, n, m, bias=g.bias, h=h)
        hs.append(h)
    torch.cuda.synchronize()
    # every (batch, head) as one of B*H heads of a single batch: [1, B*H, S, d]
    got = torch.stack(hs, dim=2).reshape(1, B * H, S8, dv)
    seq = lambda t: t[:S8].permute(1, 2, 0, 3).reshape(1, B * H, S8, -1).contiguous()
    seq_g = lambda t: t[:S8].permute(1, 2, 0).reshape(1, B * H, S8).contiguous()
    bias = None if d.bias is None else d.bias.repeat(B).contiguous()
    ref = oracle.mlstm_fwd(seq(d.q), seq(d.k), seq(d.v), seq_g(d.i_pre), seq_g(d.f_pre), None, bias)
    assert slice_err(cpu(got), ref[0]) < TOL[torch.bfloat16]
    st = (C.reshape(1, B * H, 1, dqk, dv), n.reshape(1, B * H, dqk), m.reshape(1, B * H))
    check_state(st, ref[1:], TOL[torch.bfloat16])


@pytest.mark.parametrize("dt,dqk,dv", [(torch.bfloat16, 256, 512), (torch.float32, 64, 64)],
                         ids=["bf16_256x512", "f32_64x64"])
def test_largest_admissible_slice_sampled(gpu, dt, dqk, dv):
    """One (batch, head) as long as the boundary admits: T x max(d_qk, d_v)
    elements just under 2^31 bytes, and T not a multiple of the chunk.  A
    forget preactivation of -80 at a few tokens erases the memory there (the
    old state is scaled by sigma(-80) < 1e-34), so the oracle can follow the
    window after each such token from a zero state.  Compared: the outputs
    in every window, and the final state after the last one.  The windows sit
    at the start, across superchunk boundaries, across the 2^30-byte mark of
    the widest tensor, far into the sequence and at its ragged end."""
    es = 2 if dt == torch.bfloat16 else 4
    d = max(dqk, dv)
    T = (1 << 31) // (d * es) - 64 - 23
    W = 320
    dev = torch.device(gpu)
    g = torch.Generator(device=dev).manual_seed(7001 + dqk)
    q = torch.randn(1, 1, T, dqk, generator=g, device=dev).to(dt)
    k = (torch.randn(1, 1, T, dqk, generator=g, device=dev) * dqk ** -0.5).to(dt)
    v = torch.randn(1, 1, T, dv, generator=g, device=dev).to(dt)
    i_pre = torch.randn(1, 1, T, generator=g, device=dev).to(dt)
    f_pre = (torch.randn(1, 1, T, generator=g, device=dev) + 3.0).to(dt)
    bias = torch.tensor([0.3], device=dev)
    starts = [0, 1024 - 100, (1 << 30) // (d * es) - 150, 1024 * 1500 - 37, T - W]
    for r in starts[1:]:
        f_pre[0, 0, r] = -80.0
    print("T=%d d_qk=%d d_v=%s windows at %s" % (T, dqk, dv, starts), flush=True)
    h, st = mlstm.chunkwise_fwd(q, k, v, i_pre, f_pre, None, bias,
                                state_out=(torch.empty(1, 1, 1, dqk, dv, device=dev),
                                           torch.empty(1, 1, dqk, device=dev), torch.empty(1, 1, device=dev)))
    torch.cuda.synchronize()
    b = cpu(bias)
    for r in starts:
        w = slice(r, r + W)
        ref = oracle.mlstm_fwd(cpu(q[:, :, w]), cpu(k[:, :, w]), cpu(v[:, :, w]), cpu(i_pre[:, :, w]),
                               cpu(f_pre[:, :, w]), None, b)
        assert slice_err(cpu(h[:, :, w]), ref[0]) < TOL[dt], r
    check_state(st, ref[1:], TOL[dt])
