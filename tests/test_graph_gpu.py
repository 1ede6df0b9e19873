"""HIP-graph capture of the library's calls: decode steps (mLSTM and
retention, state updated in place) and a chunkwise prefill, captured through
the C ABI on torch's capture stream and replayed several times, with eager
work and synchronisations between the replays.  Every replay must equal
eager calls of the same steps from the same state, bit for bit (same kernels,
same inputs).  The library issues no allocation, memset or synchronisation
inside these calls, so a serving loop can capture them."""
import pytest
import torch

from linear_recurrent_sequence_mlstm_amd import _lib as mlstm
from linear_recurrent_sequence_mlstm_amd.workloads import workload

pytestmark = pytest.mark.gpu

S = 8  # steps per captured graph


def _eager_noise(dev):
    # unrelated eager work between replays
    x = torch.randn(4096, device=dev)
    return float((x * 2).sum())


def test_mlstm_decode_steps_replayed_from_a_graph(gpu):
    d = workload("xlstm7b_decode_B256", B=4, steps=S).to(gpu)
    _, B, H, dqk = d.q.shape
    dv = d.v.shape[-1]
    C = torch.zeros(B, H, 1, dqk, dv, device=gpu)
    n = torch.zeros(B, H, dqk, device=gpu)
    m = torch.zeros(B, H, device=gpu)
    hg = [torch.empty(B, H, dv, dtype=d.q.dtype, device=gpu) for _ in range(S)]
    mlstm.lib()  # load before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(S):
            mlstm.step(d.q[s], d.k[s], d.v[s], d.i_pre[s], d.f_pre[s], C, n, m, bias=d.bias, h=hg[s])
    for rep in range(3):
        Ce, ne, me = C.clone(), n.clone(), m.clone()
        graph.replay()
        he = [mlstm.step(d.q[s], d.k[s], d.v[s], d.i_pre[s], d.f_pre[s], Ce, ne, me, bias=d.bias)
              for s in range(S)]
        torch.cuda.synchronize()
        for s in range(S):
            assert torch.equal(hg[s], he[s]), (rep, s)
        assert torch.equal(C, Ce) and torch.equal(n, ne) and torch.equal(m, me), rep
        _eager_noise(gpu)
        torch.cuda.synchronize()


def test_retention_decode_steps_replayed_from_a_graph(gpu):
    q, k, v = workload("retnet_msr_T2048", B=2, T=S)
    q, k, v = (t.to(gpu) for t in (q, k, v))
    B, H, _, dk = q.shape
    dv = v.shape[-1]
    St = torch.randn(B, H, dk, dv, device=gpu) * 0.1
    og = [torch.empty(B, H, dv, dtype=q.dtype, device=gpu) for _ in range(S)]
    toks = [tuple(t[:, :, s].contiguous() for t in (q, k, v)) for s in range(S)]
    mlstm.lib()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(S):
            mlstm.retention_step(*toks[s], St, out=og[s])
    for rep in range(3):
        Se = St.clone()
        graph.replay()
        oe = [mlstm.retention_step(*toks[s], Se) for s in range(S)]
        torch.cuda.synchronize()
        for s in range(S):
            assert torch.equal(og[s], oe[s]), (rep, s)
        assert torch.equal(St, Se), rep
        _eager_noise(gpu)
        torch.cuda.synchronize()


def test_chunkwise_prefill_replayed_from_a_graph(gpu):
    x = workload("xlstm7b_prefill_T8192", T=700, H=2).to(gpu)
    B, H, T, dqk = x.q.shape
    dv = x.v.shape[-1]
    ws = torch.empty(mlstm.chunkwise_workspace_bytes(B, H, T, dqk, dv, dtype=x.q.dtype), dtype=torch.uint8,
                     device=gpu)
    h = torch.empty(B, H, T, dv, dtype=x.q.dtype, device=gpu)
    st = (torch.empty(B, H, 1, dqk, dv, device=gpu), torch.empty(B, H, dqk, device=gpu),
          torch.empty(B, H, device=gpu))
    mlstm.lib()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mlstm.chunkwise_fwd(x.q, x.k, x.v, x.i_pre, x.f_pre, x.o_pre, x.bias, h=h, state_out=st, workspace=ws)
    he, ste = mlstm.chunkwise_fwd(x.q, x.k, x.v, x.i_pre, x.f_pre, x.o_pre, x.bias)
    for rep in range(3):
        h.zero_()
        for t in st:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, he), rep
        for a, b in zip(st, ste):
            assert torch.equal(a, b), rep
        _eager_noise(gpu)
