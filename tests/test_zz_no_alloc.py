"""The no-allocation forward entry point (mlstm_chunkwise_fwd_noalloc, for
callers that cannot allocate device memory) against the workspace entry
point it shares its kernels with: two calls in a row, the second one smaller,
so that the second finds the first call's leftovers in the scratch array.
The outputs must be identical (the same kernels on the same inputs)."""
import pytest
import torch

from linear_recurrent_sequence_mlstm_amd import _lib as mlstm
from linear_recurrent_sequence_mlstm_amd.workloads import mlstm_inputs, workload

pytestmark = pytest.mark.gpu


def _both(x, dev, nb=1, norm_mode="vector"):
    g = x.to(dev)
    B, H, T, dqk = g.q.shape
    dv = g.v.shape[-1]
    st = torch.Generator().manual_seed(T)
    C0 = (torch.randn(B, H, nb, dqk // nb, dv // nb, generator=st) * 0.3).to(dev)
    n0 = (torch.randn(B, H, dqk, generator=st) * 0.3).to(dev)
    m0 = (torch.rand(B, H, generator=st) * 2 - 1).to(dev)
    h_ref, s_ref = mlstm.chunkwise_fwd(g.q, g.k, g.v, g.i_pre, g.f_pre, g.o_pre, g.bias, state=(C0, n0, m0),
                                       num_blocks=nb, norm_mode=norm_mode)
    h = torch.full_like(h_ref, float("nan"))
    s_out = tuple(torch.full_like(t, float("nan")) for t in s_ref)
    mlstm.chunkwise_fwd_noalloc(g.q, g.k, g.v, g.i_pre, g.f_pre, h, s_out, g.o_pre, g.bias, state=(C0, n0, m0),
                                num_blocks=nb, norm_mode=norm_mode)
    torch.cuda.synchronize()
    assert torch.equal(h, h_ref)
    for a, b in zip(s_out, s_ref):
        assert torch.equal(a, b)


def test_noalloc_matches_workspace_entry_point(gpu):
    print("noalloc: 7B prefill shape B=1 H=8 T=8192, then a smaller ragged call", flush=True)
    _both(workload("xlstm7b_prefill_T8192"), gpu)
    x = mlstm_inputs(2, 2, 333, 64, 128, seed=5, dtype="bf16", k_scale=1 / 8, f_mix=True, with_o=True,
                     bias="uniform")
    _both(x, gpu)
    print("noalloc: two memory blocks, per-block normaliser", flush=True)
    x = mlstm_inputs(1, 2, 777, 64, 64, seed=6, dtype="bf16", nb=2, k_scale=1 / 8, f_mix=True, bias="uniform")
    _both(x, gpu, nb=2, norm_mode="block")
