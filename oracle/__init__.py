"""fp64 CPU oracle for the mLSTM recurrence and RetNet retention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the package smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may import
this module.  The GPU library (``linear_recurrent_sequence_mlstm_amd``) never
imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, one sequential loop over
time per (batch, head), OpenMP across the independent (batch, head) pairs).
This wrapper only converts inputs to contiguous float64 arrays, allocates the
outputs and calls the C entry points through ctypes.  Inputs given as torch
tensors (bf16 or fp32) are upcast exactly, so the oracle sees the very values
the GPU receives.

Parity status of each function (what pins it is listed in the tests):
  mlstm_fwd        pinned (brute-force quadratic form, unstabilised direct
                   recurrence, stabiliser-shift invariance, linear-attention
                   special case, T=1 closed form, state carry)
  mlstm_step       pinned (equals mlstm_fwd one token at a time, T=1 form)
  retention_fwd    pinned (decay-matrix closed form of the RetNet page)
  groupnorm        pinned (torch's group_norm in fp64; zero mean and
                   var/(var+eps) variance of every normalised row)
  mlstm_bwd        pinned (central finite differences of mlstm_fwd for every
                   input, also with a loss on the final state; torch autograd
                   through an unstabilised fp64 recurrence written in the
                   test; a split run chained through the state gradients;
                   the per-token bias terms against their closed form)
  retention_bwd    pinned (central finite differences of retention_fwd;
                   torch autograd through the decay-matrix parallel form)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False, out: str | None = None, extra_flags=()) -> str:
    """Compile oracle.c with gcc into a shared library; returns its path."""
    out = out or _LIB
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(_SRC):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
           *extra_flags, _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _load(path: str | None = None):
    global _lib
    if path is None and _lib is not None:
        return _lib
    lib = ctypes.CDLL(path or build())
    P = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.oracle_mlstm_fwd.argtypes = [i, i, i, i, i, i, i] + [P] * 14
    lib.oracle_mlstm_fwd.restype = i
    lib.oracle_mlstm_step.argtypes = [i, i, i, i, i, i] + [P] * 11
    lib.oracle_mlstm_step.restype = i
    lib.oracle_retention_fwd.argtypes = [i, i, i, i, i] + [P] * 7
    lib.oracle_retention_fwd.restype = i
    lib.oracle_mlstm_bwd.argtypes = [i, i, i, i, i, i] + [P] * 24
    lib.oracle_mlstm_bwd.restype = i
    lib.oracle_retention_bwd.argtypes = [i, i, i, i, i] + [P] * 11
    lib.oracle_retention_bwd.restype = i
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i
    if path is None:
        _lib = lib
    return lib


def _f64(x):
    """Contiguous float64 numpy copy of a numpy array or torch tensor (or None)."""
    if x is None:
        return None
    if "torch" in sys.modules:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float64).numpy())
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    return _load().oracle_num_threads()


# normaliser readings (see oracle.c, cell_step): the vector n . q used
# throughout, the scalar n = f n + i the XLSTMv2 page prints, and a
# per-block vector normaliser for the block-diagonal memory
NORM_MODES = {"vector": 1, "scalar": 2, "block": 3}


def mlstm_fwd(q, k, v, i_pre, f_pre, o_pre=None, bias=None, C0=None, n0=None,
              m0=None, num_blocks=1, normalise=True, m_shift=None, lib=None,
              norm_mode="vector"):
    """Sequence form.  Shapes: q,k [B,H,T,dqk]; v [B,H,T,dv]; gates [B,H,T];
    o_pre [B,H,T,dv] or None; bias [H] or None; C0 [B,H,nb,dqk/nb,dv/nb];
    n0 [B,H,dqk] ([B,H] with norm_mode "scalar"); m0 [B,H].
    Returns (h, C, n, m) as float64 arrays (n [B,H] in scalar mode)."""
    q, k, v, ip, fp = map(_f64, (q, k, v, i_pre, f_pre))
    op, bs, c0, nn0, mm0, ms = map(_f64, (o_pre, bias, C0, n0, m0, m_shift))
    B, H, T, dqk = q.shape
    mode = NORM_MODES[norm_mode] if normalise else 0
    if mode == 2 and nn0 is not None:
        e = np.zeros((B, H, dqk))
        e[:, :, 0] = nn0.reshape(B, H)
        nn0 = e
    dv = v.shape[-1]
    nb = int(num_blocks)
    assert k.shape == q.shape and v.shape == (B, H, T, dv)
    assert ip.shape == (B, H, T) and fp.shape == (B, H, T)
    h = np.zeros((B, H, T, dv))
    C = np.zeros((B, H, nb, dqk // nb, dv // nb))
    n = np.zeros((B, H, dqk))
    m = np.zeros((B, H))
    rc = (lib or _load()).oracle_mlstm_fwd(
        B, H, T, dqk, dv, nb, mode, _ptr(q), _ptr(k), _ptr(v),
        _ptr(ip), _ptr(fp), _ptr(op), _ptr(bs), _ptr(c0), _ptr(nn0), _ptr(mm0),
        _ptr(ms), _ptr(h), _ptr(C), _ptr(n), _ptr(m))
    if rc != 0:
        raise ValueError("oracle_mlstm_fwd failed with %d" % rc)
    return h, C, (n[:, :, 0].copy() if mode == 2 else n), m


def mlstm_step(q, k, v, i_pre, f_pre, C, n, m, o_pre=None, bias=None,
               num_blocks=1, lib=None, norm_mode="vector"):
    """One decode step.  q,k [B,H,dqk]; v [B,H,dv]; gates [B,H]; C,n,m are
    float64 arrays updated IN PLACE (n [B,H] with norm_mode "scalar").
    Returns h [B,H,dv] (float64)."""
    q, k, v, ip, fp, op, bs = map(_f64, (q, k, v, i_pre, f_pre, o_pre, bias))
    for a in (C, n, m):
        assert isinstance(a, np.ndarray) and a.dtype == np.float64 and a.flags.c_contiguous
    B, H, dqk = q.shape
    dv = v.shape[-1]
    mode = NORM_MODES[norm_mode]
    nn = n
    if mode == 2:
        nn = np.zeros((B, H, dqk))
        nn[:, :, 0] = n.reshape(B, H)
    h = np.zeros((B, H, dv))
    rc = (lib or _load()).oracle_mlstm_step(
        B, H, dqk, dv, int(num_blocks), mode, _ptr(q), _ptr(k), _ptr(v), _ptr(ip),
        _ptr(fp), _ptr(op), _ptr(bs), _ptr(C), _ptr(nn), _ptr(m), _ptr(h))
    if rc != 0:
        raise ValueError("oracle_mlstm_step failed with %d" % rc)
    if mode == 2:
        n.reshape(B, H)[...] = nn[:, :, 0]
    return h


def groupnorm(y, weight=None, bias=None, eps=1e-5):
    """Per-head group norm of retention outputs ("Multi-Scale Retention
    (MSR)" section of the "Edifice.Attention.RetNet" page: a group norm
    normalises each head's output).  y [B,H,T,dv]; one group per head over
    its dv channels, per token: (y - mean) / sqrt(var + eps) with the mean
    and biased variance over those dv values, then the per-channel affine
    weight, bias [H*dv] (None: 1, 0).  Plain numpy in fp64."""
    y = _f64(y)
    B, H, T, dv = y.shape
    mean = y.mean(axis=3, keepdims=True)
    var = ((y - mean) ** 2).mean(axis=3, keepdims=True)
    out = (y - mean) / np.sqrt(var + eps)
    if weight is not None:
        out = out * _f64(weight).reshape(1, H, 1, dv)
    if bias is not None:
        out = out + _f64(bias).reshape(1, H, 1, dv)
    return out


def retention_fwd(q, k, v, gamma=None, S0=None, lib=None):
    """Retention recurrence.  q,k [B,H,T,dk]; v [B,H,T,dv]; gamma [H] or None
    (then 1 - 2^(-5-h)); S0 [B,H,dk,dv] or None.  Returns (out, S)."""
    q, k, v, g, s0 = map(_f64, (q, k, v, gamma, S0))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    out = np.zeros((B, H, T, dv))
    S = np.zeros((B, H, dk, dv))
    rc = (lib or _load()).oracle_retention_fwd(
        B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s0),
        _ptr(out), _ptr(S))
    if rc != 0:
        raise ValueError("oracle_retention_fwd failed with %d" % rc)
    return out, S


def mlstm_bwd(q, k, v, i_pre, f_pre, dh, o_pre=None, bias=None, C0=None, n0=None,
              m0=None, lib=None, num_blocks=1, dCT=None, dnT=None):
    """Gradients of sum(dh * h) for the mLSTM sequence form (vector
    normaliser; num_blocks memory blocks), h = mlstm_fwd(q, k, v, ...)[0].  Shapes as
    in mlstm_fwd; dh [B,H,T,dv].  dCT (shaped as C0), dnT [B,H,dqk]: optional
    gradient arriving at the stabilised final state (S~_T, n~_T at fixed m_T).
    Returns a dict of float64 arrays: dq, dk, dv, di (i_pre), df (f_pre), do
    (o_pre; None without o_pre), dbias [H], dbias_t [B,H,T] (the per-token
    terms of dbias), z [B,H,T] (n_t . q_t + bias in true units: the gradient
    jumps where |z| crosses 1), dC0 [B,H,dqk,dv] and dn0 [B,H,dqk]
    (gradients of the stabilised initial state, zero-state runs included)."""
    q, k, v, ip, fp, g = map(_f64, (q, k, v, i_pre, f_pre, dh))
    op, bs, c0, nn0, mm0, dct, dnt = map(_f64, (o_pre, bias, C0, n0, m0, dCT, dnT))
    B, H, T, dqk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape == (B, H, T, dv) and g.shape == v.shape
    nb = int(num_blocks)
    cshape = (B, H, dqk, dv) if nb == 1 else (B, H, nb, dqk // nb, dv // nb)
    if c0 is not None:
        c0 = np.ascontiguousarray(c0.reshape(cshape))
    if dct is not None:
        dct = np.ascontiguousarray(dct.reshape(cshape))
    if dnt is not None:
        assert dnt.shape == (B, H, dqk)
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               di=np.zeros((B, H, T)), df=np.zeros((B, H, T)),
               do=np.zeros_like(v) if op is not None else None,
               dbias=np.zeros(H), dbias_t=np.zeros((B, H, T)), z=np.zeros((B, H, T)), dC0=np.zeros(cshape),
               dn0=np.zeros((B, H, dqk)))
    rc = (lib or _load()).oracle_mlstm_bwd(
        B, H, T, dqk, dv, nb, _ptr(q), _ptr(k), _ptr(v), _ptr(ip), _ptr(fp), _ptr(op),
        _ptr(bs), _ptr(c0), _ptr(nn0), _ptr(mm0), _ptr(g), _ptr(dct), _ptr(dnt), _ptr(out["dq"]),
        _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["di"]), _ptr(out["df"]),
        _ptr(out["do"]), _ptr(out["dbias"]), _ptr(out["dbias_t"]), _ptr(out["z"]), _ptr(out["dC0"]), _ptr(out["dn0"]))
    if rc != 0:
        raise ValueError("oracle_mlstm_bwd failed with %d" % rc)
    return out


def retention_bwd(q, k, v, dout, gamma=None, S0=None, lib=None, dS_T=None):
    """Gradients of sum(dout * out) (+ <dS_T, S_T> with the optional gradient
    dS_T [B,H,dk,dv] arriving at the final state) for out, S_T =
    retention_fwd(q, k, v, gamma, S0).  Returns a dict of float64 arrays dq,
    dk, dv and dS0 [B,H,dk,dv]."""
    q, k, v, g, s0, go, dst = map(_f64, (q, k, v, gamma, S0, dout, dS_T))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v), dS0=np.zeros((B, H, dk, dv)))
    rc = (lib or _load()).oracle_retention_bwd(
        B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s0), _ptr(go), _ptr(dst), _ptr(out["dq"]),
        _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dS0"]))
    if rc != 0:
        raise ValueError("oracle_retention_bwd failed with %d" % rc)
    return out
