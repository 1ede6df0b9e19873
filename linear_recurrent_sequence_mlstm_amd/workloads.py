"""Seeded synthetic inputs for the mLSTM / retention hot path.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic.  Both the GPU tests / benchmark and the CPU oracle
consume the tensors it returns (the oracle upcasts them exactly), so the two
sides always see bit-identical inputs.

Draw order is fixed per workload: q, k, v, input-gate preactivation,
forget-gate preactivation, output-gate preactivation, normaliser bias.
Everything is drawn in fp32 on the CPU from ``torch.Generator().manual_seed``
and then cast (round-to-nearest-even) to the workload's dtype.

Workloads (shapes and distributions follow the pages' configurations):
  cell_fp32_T60          single cell, fp32, B=1 H=4 d_qk=d_v=64 T=60
  retnet_msr_T2048       RetNet multi-scale retention, bf16, B=8 H=4 d=64 T=2048
  xlstm7b_prefill_T8192  xLSTM-7B-shaped layer, bf16, B=1 H=8 d_qk=256 d_v=512 T=8192
  xlstm7b_decode_B256    xLSTM-7B-shaped decode, bf16 tokens, B=256 H=8, 128 steps
  xlstm2_blockdiag_T65536 xLSTM-v2 block-diagonal, bf16, B=4 H=4 d=64 nb=2 T=65536
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

# name -> (seed, dict of generator arguments)
WORKLOADS = {
    "cell_fp32_T60": dict(seed=1001, B=1, H=4, T=60, dqk=64, dv=64, nb=1,
                          dtype="f32", k_scale=1.0 / 8, f_mean=3.0, with_o=True,
                          bias="zero", chunk=64),
    "retnet_msr_T2048": dict(seed=1002, B=8, H=4, T=2048, dqk=64, dv=64, nb=1,
                             dtype="bf16", qkv_scale=1.0 / 8, chunk=64),
    "xlstm7b_prefill_T8192": dict(seed=1003, B=1, H=8, T=8192, dqk=256, dv=512,
                                  nb=1, dtype="bf16", k_scale=1.0 / 16,
                                  f_mean=3.0, chunk=64),
    "xlstm7b_decode_B256": dict(seed=1004, B=256, H=8, steps=128, dqk=256,
                                dv=512, nb=1, dtype="bf16", k_scale=1.0 / 16,
                                f_mean=3.0),
    "xlstm2_blockdiag_T65536": dict(seed=1005, B=4, H=4, T=65536, dqk=64, dv=64,
                                    nb=2, dtype="bf16", k_scale=1.0 / 8,
                                    f_mix=True, bias="uniform", chunk=64),
}

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class MlstmInputs:
    """Sequence inputs.  q,k [B,H,T,dqk]; v [B,H,T,dv]; i_pre,f_pre [B,H,T];
    o_pre [B,H,T,dv] or None; bias [H] fp32 or None."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    i_pre: torch.Tensor
    f_pre: torch.Tensor
    o_pre: Optional[torch.Tensor] = None
    bias: Optional[torch.Tensor] = None
    num_blocks: int = 1
    chunk: int = 64
    meta: dict = field(default_factory=dict)

    def to(self, device):
        mv = lambda t: None if t is None else t.to(device).contiguous()
        return MlstmInputs(mv(self.q), mv(self.k), mv(self.v), mv(self.i_pre),
                           mv(self.f_pre), mv(self.o_pre), mv(self.bias),
                           self.num_blocks, self.chunk, dict(self.meta))


def mlstm_inputs(B, H, T, dqk, dv, *, seed, dtype="bf16", nb=1, k_scale=1.0,
                 f_mean=3.0, f_mix=False, with_o=False, bias=None, chunk=64,
                 i_mean=0.0) -> MlstmInputs:
    """Draw one set of sequence inputs.

    k is multiplied by ``k_scale`` before the cast.  The forget preactivation
    is N(f_mean, 1), or with ``f_mix`` a per-token mixture: 80 % N(4, 1) and
    20 % N(-2, 1) (Bernoulli draw first, then both normals).  ``bias`` is
    None (absent), "zero" or "uniform" (U(-0.5, 0.5) per head, fp32).
    """
    g = torch.Generator().manual_seed(int(seed))
    dt = _DT[dtype]
    q = torch.randn(B, H, T, dqk, generator=g)
    k = torch.randn(B, H, T, dqk, generator=g) * k_scale
    v = torch.randn(B, H, T, dv, generator=g)
    i_pre = torch.randn(B, H, T, generator=g) + i_mean
    if f_mix:
        sel = torch.rand(B, H, T, generator=g) < 0.8
        hi = torch.randn(B, H, T, generator=g) + 4.0
        lo = torch.randn(B, H, T, generator=g) - 2.0
        f_pre = torch.where(sel, hi, lo)
    else:
        f_pre = torch.randn(B, H, T, generator=g) + f_mean
    o_pre = torch.randn(B, H, T, dv, generator=g) if with_o else None
    if bias == "uniform":
        bias_t = torch.rand(H, generator=g) - 0.5
    elif bias == "zero":
        bias_t = torch.zeros(H)
    else:
        bias_t = None
    cast = lambda t: None if t is None else t.to(dt).contiguous()
    return MlstmInputs(cast(q), cast(k), cast(v), cast(i_pre), cast(f_pre),
                       cast(o_pre), bias_t, nb, chunk,
                       dict(B=B, H=H, T=T, dqk=dqk, dv=dv, dtype=dtype, seed=seed))


def retention_inputs(B, H, T, dk, dv, *, seed, dtype="bf16", qkv_scale=1.0 / 8):
    """Q, K, V ~ N(0,1) * qkv_scale, cast to dtype.  Returns (q, k, v)."""
    g = torch.Generator().manual_seed(int(seed))
    dt = _DT[dtype]
    q = (torch.randn(B, H, T, dk, generator=g) * qkv_scale).to(dt)
    k = (torch.randn(B, H, T, dk, generator=g) * qkv_scale).to(dt)
    v = (torch.randn(B, H, T, dv, generator=g) * qkv_scale).to(dt)
    return q, k, v


@dataclass
class DecodeInputs:
    """Per-step tokens for the decode workload.  q,k [S,B,H,dqk];
    v [S,B,H,dv]; i_pre,f_pre [S,B,H]; o_pre [S,B,H,dv] or None; bias [H]."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    i_pre: torch.Tensor
    f_pre: torch.Tensor
    o_pre: Optional[torch.Tensor] = None
    bias: Optional[torch.Tensor] = None
    num_blocks: int = 1

    def to(self, device):
        mv = lambda t: None if t is None else t.to(device).contiguous()
        return DecodeInputs(mv(self.q), mv(self.k), mv(self.v), mv(self.i_pre),
                            mv(self.f_pre), mv(self.o_pre), mv(self.bias),
                            self.num_blocks)


def decode_inputs(steps, B, H, dqk, dv, *, seed, dtype="bf16", nb=1,
                  k_scale=1.0, f_mean=3.0, with_o=False, bias=None) -> DecodeInputs:
    """A fresh token per step for every sequence; same distributions as
    :func:`mlstm_inputs` (forget preactivation N(f_mean, 1))."""
    g = torch.Generator().manual_seed(int(seed))
    dt = _DT[dtype]
    q = torch.randn(steps, B, H, dqk, generator=g)
    k = torch.randn(steps, B, H, dqk, generator=g) * k_scale
    v = torch.randn(steps, B, H, dv, generator=g)
    i_pre = torch.randn(steps, B, H, generator=g)
    f_pre = torch.randn(steps, B, H, generator=g) + f_mean
    o_pre = torch.randn(steps, B, H, dv, generator=g) if with_o else None
    if bias == "uniform":
        bias_t = torch.rand(H, generator=g) - 0.5
    elif bias == "zero":
        bias_t = torch.zeros(H)
    else:
        bias_t = None
    cast = lambda t: None if t is None else t.to(dt).contiguous()
    return DecodeInputs(cast(q), cast(k), cast(v), cast(i_pre), cast(f_pre),
                        cast(o_pre), bias_t, nb)


def workload(name: str, **override):
    """Inputs of a named workload; keyword overrides (e.g. T=512, B=2) shrink
    it for tests while keeping its distributions."""
    spec = dict(WORKLOADS[name])
    spec.update(override)
    seed = spec.pop("seed")
    if name.startswith("retnet"):
        return retention_inputs(spec["B"], spec["H"], spec["T"], spec["dqk"],
                                spec["dv"], seed=seed, dtype=spec["dtype"],
                                qkv_scale=spec["qkv_scale"])
    if "steps" in spec:
        return decode_inputs(spec["steps"], spec["B"], spec["H"], spec["dqk"],
                             spec["dv"], seed=seed, dtype=spec["dtype"],
                             nb=spec["nb"], k_scale=spec["k_scale"],
                             f_mean=spec["f_mean"], with_o=spec.get("with_o", False),
                             bias=spec.get("bias"))
    return mlstm_inputs(spec["B"], spec["H"], spec["T"], spec["dqk"], spec["dv"],
                        seed=seed, dtype=spec["dtype"], nb=spec["nb"],
                        k_scale=spec["k_scale"], f_mean=spec.get("f_mean", 3.0),
                        f_mix=spec.get("f_mix", False),
                        with_o=spec.get("with_o", False), bias=spec.get("bias"),
                        chunk=spec.get("chunk", 64))


def grad_output(shape, *, seed, dtype="bf16", scale=1.0) -> torch.Tensor:
    """Seeded incoming gradient dh ~ N(0, 1) * scale of the given shape, cast
    to dtype (the loss sum(dh * h) of a backward pass)."""
    g = torch.Generator().manual_seed(int(seed))
    return (torch.randn(*shape, generator=g) * scale).to(_DT[dtype]).contiguous()
