"""ctypes binding of libmlstm.so (C ABI in include/mlstm.h).

Argument marshalling only: checks devices, dtypes, shapes and contiguity,
allocates outputs and workspace as torch tensors (PyTorch provides device
memory and the current stream), and calls the C entry points.  Every step of
the computation runs in the HIP kernels; there is no fallback path, and a
missing library raises an error.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmlstm.so")
_lib = None

F32, BF16 = 0, 1
_DT = {torch.float32: F32, torch.bfloat16: BF16}

# Every symbol declared in include/mlstm.h.
EXPORTS = ("mlstm_abi_version", "mlstm_last_error", "mlstm_set_profile_events",
           "mlstm_chunkwise_workspace_bytes",
           "mlstm_chunkwise_fwd", "mlstm_chunkwise_fwd_ex", "mlstm_step", "mlstm_step_ex",
           "retention_chunkwise_workspace_bytes",
           "retention_chunkwise_fwd", "retention_chunkwise_groupnorm_workspace_bytes",
           "retention_chunkwise_groupnorm_fwd", "retention_step",
           "mlstm_chunkwise_bwd_workspace_bytes", "mlstm_chunkwise_bwd",
           "retention_chunkwise_bwd_workspace_bytes", "retention_chunkwise_bwd",
           "mlstm_chunkwise_fwd_noalloc", "mlstm_noalloc_scratch_bytes")


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libmlstm.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libmlstm.so is not built (%s); run `python -m "
                           "linear_recurrent_sequence_mlstm_amd.build`" % _LIB_PATH)
    L = ctypes.CDLL(_LIB_PATH)
    i, sz, vp, fp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p
    L.mlstm_abi_version.argtypes = []
    L.mlstm_abi_version.restype = i
    L.mlstm_last_error.argtypes = []
    L.mlstm_last_error.restype = ctypes.c_char_p
    L.mlstm_set_profile_events.argtypes = [vp, vp]
    L.mlstm_set_profile_events.restype = i
    L.mlstm_chunkwise_workspace_bytes.argtypes = [i] * 7 + [i]
    L.mlstm_chunkwise_workspace_bytes.restype = sz
    L.mlstm_chunkwise_fwd.argtypes = [i] * 8 + [vp] * 6 + [fp] * 7 + [vp, vp, sz, vp]
    L.mlstm_chunkwise_fwd.restype = i
    L.mlstm_step.argtypes = [i] * 6 + [vp] * 6 + [fp] * 4 + [vp, vp]
    L.mlstm_step.restype = i
    L.mlstm_chunkwise_fwd_ex.argtypes = [i] * 9 + [vp] * 6 + [fp] * 7 + [vp, vp, sz, vp]
    L.mlstm_chunkwise_fwd_ex.restype = i
    L.mlstm_chunkwise_fwd_noalloc.argtypes = [i] * 9 + [vp] * 6 + [fp] * 7 + [vp, vp]
    L.mlstm_chunkwise_fwd_noalloc.restype = i
    L.mlstm_noalloc_scratch_bytes.argtypes = []
    L.mlstm_noalloc_scratch_bytes.restype = sz
    L.mlstm_step_ex.argtypes = [i] * 7 + [vp] * 6 + [fp] * 4 + [vp, vp]
    L.mlstm_step_ex.restype = i
    L.retention_chunkwise_workspace_bytes.argtypes = [i] * 6 + [i]
    L.retention_chunkwise_workspace_bytes.restype = sz
    L.retention_chunkwise_fwd.argtypes = [i] * 7 + [vp] * 3 + [fp] * 3 + [vp, vp, sz, vp]
    L.retention_chunkwise_fwd.restype = i
    L.retention_chunkwise_groupnorm_workspace_bytes.argtypes = [i] * 6 + [i]
    L.retention_chunkwise_groupnorm_workspace_bytes.restype = sz
    L.retention_chunkwise_groupnorm_fwd.argtypes = ([i] * 7 + [vp] * 3 + [fp] * 5 + [ctypes.c_float] +
                                                    [vp, vp, sz, vp])
    L.retention_chunkwise_groupnorm_fwd.restype = i
    L.retention_step.argtypes = [i] * 5 + [vp] * 3 + [fp] * 2 + [vp, vp]
    L.retention_step.restype = i
    L.mlstm_chunkwise_bwd_workspace_bytes.argtypes = [i] * 8
    L.mlstm_chunkwise_bwd_workspace_bytes.restype = sz
    L.mlstm_chunkwise_bwd.argtypes = ([i] * 8 + [vp] * 6 + [fp] * 4 + [vp] + [fp] * 2 + [vp] * 6 + [fp] * 3 +
                                      [vp, sz, vp])
    L.mlstm_chunkwise_bwd.restype = i
    L.retention_chunkwise_bwd_workspace_bytes.argtypes = [i] * 7
    L.retention_chunkwise_bwd_workspace_bytes.restype = sz
    L.retention_chunkwise_bwd.argtypes = [i] * 7 + [vp] * 3 + [fp] * 2 + [vp] + [fp] + [vp] * 3 + [fp] + [vp, sz, vp]
    L.retention_chunkwise_bwd.restype = i
    _lib = L
    return L


def abi_version() -> int:
    return lib().mlstm_abi_version()


def last_error() -> str:
    return lib().mlstm_last_error().decode()


def set_profile_events(ev_start=None, ev_stop=None):
    """Record two torch.cuda.Event objects (enable_timing=True) around the
    main kernel of every following chunkwise call on this thread; call with
    no arguments to stop."""
    h0 = h1 = None
    if ev_start is not None:
        for ev in (ev_start, ev_stop):
            if ev.cuda_event == 0:  # torch creates the HIP event on first record
                ev.record()
        h0, h1 = ctypes.c_void_p(ev_start.cuda_event), ctypes.c_void_p(ev_stop.cuda_event)
    _check(lib().mlstm_set_profile_events(h0, h1), "mlstm_set_profile_events")


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError("%s failed (%d): %s" % (what, rc, last_error()))


def _ptr(t):
    # a plain int: ctypes turns it into the void* argument without an object
    return None if t is None else t.data_ptr()


def _need(t, name, shape, dtype, device):
    if t is None:
        return
    # the common case in one expression (a call checks about a dozen tensors,
    # and these checks dominated the host time of a short call); any failure
    # falls through to the checks below, which name what is wrong
    if isinstance(t, torch.Tensor) and t.dtype is dtype and t.shape == shape and t.is_contiguous() \
            and t.device == device:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device):
    """The current stream of `device` as a raw hipStream_t (an int)."""
    if _raw_stream is not None:
        return _raw_stream(device.index if device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def chunkwise_workspace_bytes(B, H, T, dqk, dv, num_blocks=1, chunk=64, dtype=torch.bfloat16) -> int:
    return int(lib().mlstm_chunkwise_workspace_bytes(B, H, T, dqk, dv, num_blocks, chunk, _DT[dtype]))


def retention_workspace_bytes(B, H, T, dk, dv, chunk=64, dtype=torch.bfloat16) -> int:
    return int(lib().retention_chunkwise_workspace_bytes(B, H, T, dk, dv, chunk, _DT[dtype]))


def _workspace(nbytes, device, workspace):
    """The caller's workspace (a contiguous tensor on `device`, any dtype, at
    least nbytes long) or, without one, a fresh one; returns (tensor, its size
    in bytes).  A caller's workspace that is too small raises: a caller that
    passes one does not expect the call to allocate."""
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor):
            raise TypeError("workspace must be a torch.Tensor")
        if workspace.device != device:
            raise ValueError("workspace is on %s, expected %s" % (workspace.device, device))
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        size = workspace.numel() * workspace.element_size()
        if size < nbytes:
            raise ValueError("workspace holds %d bytes, the call needs %d" % (size, nbytes))
        return workspace, size
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    return ws, ws.numel()


# normaliser readings of the _ex entry points (MLSTM_NORM_* in mlstm.h)
NORM_MODES = {"vector": 0, "scalar": 1, "block": 2}


def chunkwise_fwd(q, k, v, i_pre, f_pre, o_pre=None, bias=None, state=None, num_blocks=1,
                  chunk=64, return_state=True, h=None, state_out=None, workspace=None,
                  norm_mode="vector"):
    """mlstm_chunkwise_fwd(_ex).  q,k [B,H,T,dqk]; v [B,H,T,dv]; i_pre,f_pre [B,H,T];
    o_pre [B,H,T,dv] or None (all of one dtype, on one GPU); bias [H] fp32;
    state = (C0 [B,H,nb,dqk/nb,dv/nb], n0 [B,H,dqk] ([B,H] for norm_mode
    "scalar"), m0 [B,H]) fp32 or None.  Returns (h, (C, n, m)) or (h, None)."""
    mode = NORM_MODES[norm_mode]
    B, H, T, dqk = q.shape
    dv = v.shape[-1]
    nb = int(num_blocks)
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise TypeError("unsupported dtype %s" % dt)
    _need(k, "k", (B, H, T, dqk), dt, dev)
    _need(v, "v", (B, H, T, dv), dt, dev)
    _need(i_pre, "i_pre", (B, H, T), dt, dev)
    _need(f_pre, "f_pre", (B, H, T), dt, dev)
    _need(o_pre, "o_pre", (B, H, T, dv), dt, dev)
    _need(bias, "bias", (H,), torch.float32, dev)
    _need(q, "q", (B, H, T, dqk), dt, dev)
    scalar_n = mode == NORM_MODES["scalar"]  # n is [B,H] only for the scalar normaliser
    sshape = ((B, H, nb, dqk // nb, dv // nb), (B, H) if scalar_n else (B, H, dqk), (B, H))
    C0 = n0 = m0 = None
    if state is not None:
        C0, n0, m0 = state
        for t, nm, shp in zip((C0, n0, m0), ("C0", "n0", "m0"), sshape):
            _need(t, nm, shp, torch.float32, dev)
    if h is None:
        h = torch.empty(B, H, T, dv, dtype=dt, device=dev)
    _need(h, "h", (B, H, T, dv), dt, dev)
    Co = no = mo = None
    if return_state:
        if state_out is not None:
            Co, no, mo = state_out
        else:
            Co = torch.empty(sshape[0], dtype=torch.float32, device=dev)
            no = torch.empty(sshape[1], dtype=torch.float32, device=dev)
            mo = torch.empty(sshape[2], dtype=torch.float32, device=dev)
        for t, nm, shp in zip((Co, no, mo), ("C_out", "n_out", "m_out"), sshape):
            _need(t, nm, shp, torch.float32, dev)
    L = lib()
    nbytes = L.mlstm_chunkwise_workspace_bytes(B, H, T, dqk, dv, nb, chunk, _DT[dt])
    if nbytes == 0:
        _check(L.mlstm_chunkwise_fwd(B, H, T, dqk, dv, nb, chunk, _DT[dt], *([None] * 13),
                                     None, None, 0, None), "mlstm_chunkwise_fwd")
    ws, wsb = _workspace(nbytes, dev, workspace)
    rc = L.mlstm_chunkwise_fwd_ex(B, H, T, dqk, dv, nb, chunk, _DT[dt], mode, _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(i_pre), _ptr(f_pre), _ptr(o_pre), _ptr(bias), _ptr(C0), _ptr(n0),
                                  _ptr(m0), _ptr(Co), _ptr(no), _ptr(mo), _ptr(h), _ptr(ws),
                                  wsb, _stream(dev))
    _check(rc, "mlstm_chunkwise_fwd_ex")
    return h, ((Co, no, mo) if return_state else None)


def chunkwise_fwd_noalloc(q, k, v, i_pre, f_pre, h, state_out, o_pre=None, bias=None, state=None, num_blocks=1,
                          chunk=64, norm_mode="vector"):
    """mlstm_chunkwise_fwd_noalloc: chunkwise_fwd into caller-given outputs h
    [B,H,T,dv] and state_out = (C, n, m) (or None), using the library's
    per-GPU scratch array instead of a workspace; nothing is allocated."""
    mode = NORM_MODES[norm_mode]
    B, H, T, dqk = q.shape
    dv = v.shape[-1]
    nb = int(num_blocks)
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise TypeError("unsupported dtype %s" % dt)
    _need(k, "k", (B, H, T, dqk), dt, dev)
    _need(v, "v", (B, H, T, dv), dt, dev)
    _need(i_pre, "i_pre", (B, H, T), dt, dev)
    _need(f_pre, "f_pre", (B, H, T), dt, dev)
    _need(o_pre, "o_pre", (B, H, T, dv), dt, dev)
    _need(bias, "bias", (H,), torch.float32, dev)
    _need(h, "h", (B, H, T, dv), dt, dev)
    scalar_n = mode == NORM_MODES["scalar"]
    sshape = ((B, H, nb, dqk // nb, dv // nb), (B, H) if scalar_n else (B, H, dqk), (B, H))
    C0 = n0 = m0 = Co = no = mo = None
    if state is not None:
        C0, n0, m0 = state
        for t, nm, shp in zip((C0, n0, m0), ("C0", "n0", "m0"), sshape):
            _need(t, nm, shp, torch.float32, dev)
    if state_out is not None:
        Co, no, mo = state_out
        for t, nm, shp in zip((Co, no, mo), ("C_out", "n_out", "m_out"), sshape):
            _need(t, nm, shp, torch.float32, dev)
    rc = lib().mlstm_chunkwise_fwd_noalloc(B, H, T, dqk, dv, nb, chunk, _DT[dt], mode, _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(i_pre), _ptr(f_pre), _ptr(o_pre), _ptr(bias), _ptr(C0), _ptr(n0),
                                           _ptr(m0), _ptr(Co), _ptr(no), _ptr(mo), _ptr(h), _stream(dev))
    _check(rc, "mlstm_chunkwise_fwd_noalloc")
    return h


def step(q, k, v, i_pre, f_pre, C, n, m, o_pre=None, bias=None, num_blocks=1, h=None,
         norm_mode="vector"):
    """mlstm_step(_ex): one token per (b,h); C [B,H,nb,dqk/nb,dv/nb], n [B,H,dqk]
    ([B,H] for norm_mode "scalar"), m [B,H] fp32 are updated in place.
    Returns h [B,H,dv]."""
    mode = NORM_MODES[norm_mode]
    B, H, dqk = q.shape
    dv = v.shape[-1]
    nb = int(num_blocks)
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise TypeError("unsupported dtype %s" % dt)
    _need(k, "k", (B, H, dqk), dt, dev)
    _need(v, "v", (B, H, dv), dt, dev)
    _need(i_pre, "i_pre", (B, H), dt, dev)
    _need(f_pre, "f_pre", (B, H), dt, dev)
    _need(o_pre, "o_pre", (B, H, dv), dt, dev)
    _need(bias, "bias", (H,), torch.float32, dev)
    _need(C, "C", (B, H, nb, dqk // nb, dv // nb), torch.float32, dev)
    _need(n, "n", (B, H) if mode == NORM_MODES["scalar"] else (B, H, dqk), torch.float32, dev)
    _need(m, "m", (B, H), torch.float32, dev)
    if h is None:
        h = torch.empty(B, H, dv, dtype=dt, device=dev)
    _need(h, "h", (B, H, dv), dt, dev)
    rc = lib().mlstm_step_ex(B, H, dqk, dv, nb, _DT[dt], mode, _ptr(q), _ptr(k), _ptr(v), _ptr(i_pre),
                             _ptr(f_pre), _ptr(o_pre), _ptr(bias), _ptr(C), _ptr(n), _ptr(m), _ptr(h),
                             _stream(dev))
    _check(rc, "mlstm_step_ex")
    return h


def retention_chunkwise_fwd(q, k, v, gamma=None, S0=None, chunk=64, return_state=True, out=None,
                            S_out=None, workspace=None, groupnorm=None):
    """retention_chunkwise_fwd.  q,k [B,H,T,dk]; v [B,H,T,dv]; gamma [H] fp32
    or None (1 - 2^(-5-h)); S0 [B,H,dk,dv] fp32 or None.  Returns (out, S).
    groupnorm = (weight [H*dv] or None, bias [H*dv] or None, eps) applies the
    per-head group norm to the outputs (retention_chunkwise_groupnorm_fwd)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise TypeError("unsupported dtype %s" % dt)
    _need(k, "k", (B, H, T, dk), dt, dev)
    _need(v, "v", (B, H, T, dv), dt, dev)
    _need(gamma, "gamma", (H,), torch.float32, dev)
    _need(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty(B, H, T, dv, dtype=dt, device=dev)
    _need(out, "out", (B, H, T, dv), dt, dev)
    if return_state and S_out is None:
        S_out = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    if return_state:
        _need(S_out, "S_out", (B, H, dk, dv), torch.float32, dev)
    L = lib()
    if groupnorm is None:
        nbytes = L.retention_chunkwise_workspace_bytes(B, H, T, dk, dv, chunk, _DT[dt])
    else:
        nbytes = L.retention_chunkwise_groupnorm_workspace_bytes(B, H, T, dk, dv, chunk, _DT[dt])
    if nbytes == 0:
        if groupnorm is None:
            rc = L.retention_chunkwise_fwd(B, H, T, dk, dv, chunk, _DT[dt], *([None] * 7), None, 0, None)
        else:
            rc = L.retention_chunkwise_groupnorm_fwd(B, H, T, dk, dv, chunk, _DT[dt], *([None] * 8), None,
                                                     ctypes.c_float(1.0), None, None, 0, None)
        _check(rc, "retention_chunkwise_fwd")
    ws, wsb = _workspace(nbytes, dev, workspace)
    if groupnorm is not None:
        gw, gb, eps = groupnorm
        _need(gw, "gn_weight", (H * dv,), torch.float32, dev)
        _need(gb, "gn_bias", (H * dv,), torch.float32, dev)
        rc = L.retention_chunkwise_groupnorm_fwd(B, H, T, dk, dv, chunk, _DT[dt], _ptr(q), _ptr(k), _ptr(v),
                                                 _ptr(gamma), _ptr(S0), _ptr(S_out if return_state else None),
                                                 _ptr(gw), _ptr(gb), float(eps), _ptr(out), _ptr(ws),
                                                 wsb, _stream(dev))
        _check(rc, "retention_chunkwise_groupnorm_fwd")
        return out, (S_out if return_state else None)
    rc = L.retention_chunkwise_fwd(B, H, T, dk, dv, chunk, _DT[dt], _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(gamma), _ptr(S0), _ptr(S_out if return_state else None),
                                   _ptr(out), _ptr(ws), wsb, _stream(dev))
    _check(rc, "retention_chunkwise_fwd")
    return out, (S_out if return_state else None)


def retention_step(q, k, v, S, gamma=None, out=None):
    """retention_step: one token per (b,h); q,k [B,H,dk]; v [B,H,dv];
    S [B,H,dk,dv] fp32 updated in place (S = gamma S + k v^T); gamma [H]
    fp32 or None (1 - 2^(-5-h)).  Returns out = S^T q [B,H,dv]."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise TypeError("unsupported dtype %s" % dt)
    _need(k, "k", (B, H, dk), dt, dev)
    _need(v, "v", (B, H, dv), dt, dev)
    _need(gamma, "gamma", (H,), torch.float32, dev)
    _need(S, "S", (B, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty(B, H, dv, dtype=dt, device=dev)
    _need(out, "out", (B, H, dv), dt, dev)
    rc = lib().retention_step(B, H, dk, dv, _DT[dt], _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(S),
                              _ptr(out), _stream(dev))
    _check(rc, "retention_step")
    return out


def chunkwise_bwd(q, k, v, i_pre, f_pre, dh, o_pre=None, bias=None, state=None, chunk=64,
                  state_grad=True, workspace=None, num_blocks=1, final_grad=None):
    """mlstm_chunkwise_bwd: gradients of sum(dh * h) for h = chunkwise_fwd(q, k,
    v, i_pre, f_pre, o_pre, bias, state, num_blocks) (vector normaliser).
    final_grad = (dC_T [B,H,nb,dqk/nb,dv/nb] or None, dn_T [B,H,dqk] or None),
    fp32: gradient arriving at the final stabilised state (a following call's
    dC0, dn0).  Returns a dict with dq, dk, dv, di (i_pre), df (f_pre), do
    (o_pre, or None), dbias ([H] fp32, or None without bias) and, with
    state_grad, dC0 [B,H,nb,dqk/nb,dv/nb] and dn0 [B,H,dqk] (fp32)."""
    B, H, T, dqk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise TypeError("unsupported dtype %s" % dt)
    _need(q, "q", (B, H, T, dqk), dt, dev)
    _need(k, "k", (B, H, T, dqk), dt, dev)
    for t, nm in ((v, "v"), (dh, "dh")):
        _need(t, nm, (B, H, T, dv), dt, dev)
    _need(i_pre, "i_pre", (B, H, T), dt, dev)
    _need(f_pre, "f_pre", (B, H, T), dt, dev)
    _need(o_pre, "o_pre", (B, H, T, dv), dt, dev)
    _need(bias, "bias", (H,), torch.float32, dev)
    nb = int(num_blocks)
    cshape = (B, H, nb, dqk // nb, dv // nb)
    C0 = n0 = m0 = None
    if state is not None:
        C0, n0, m0 = state
        for t, nm, shp in zip((C0, n0, m0), ("C0", "n0", "m0"), (cshape, (B, H, dqk), (B, H))):
            _need(t, nm, shp, torch.float32, dev)
    dCT = dnT = None
    if final_grad is not None:
        dCT, dnT = final_grad
        _need(dCT, "dC_T", cshape, torch.float32, dev)
        _need(dnT, "dn_T", (B, H, dqk), torch.float32, dev)
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               di=torch.empty_like(i_pre), df=torch.empty_like(f_pre),
               do=torch.empty_like(o_pre) if o_pre is not None else None,
               dbias=torch.empty(H, dtype=torch.float32, device=dev) if bias is not None else None,
               dC0=torch.empty(cshape, dtype=torch.float32, device=dev) if state_grad else None,
               dn0=torch.empty(B, H, dqk, dtype=torch.float32, device=dev) if state_grad else None)
    L = lib()
    nbytes = L.mlstm_chunkwise_bwd_workspace_bytes(B, H, T, dqk, dv, nb, chunk, _DT[dt])
    if nbytes == 0:
        _check(L.mlstm_chunkwise_bwd(B, H, T, dqk, dv, nb, chunk, _DT[dt], *([None] * 22), None, 0, None),
               "mlstm_chunkwise_bwd")
    ws, wsb = _workspace(nbytes, dev, workspace)
    rc = L.mlstm_chunkwise_bwd(B, H, T, dqk, dv, nb, chunk, _DT[dt], _ptr(q), _ptr(k), _ptr(v), _ptr(i_pre),
                               _ptr(f_pre), _ptr(o_pre), _ptr(bias), _ptr(C0), _ptr(n0), _ptr(m0),
                               _ptr(dh), _ptr(dCT), _ptr(dnT), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                               _ptr(out["di"]),
                               _ptr(out["df"]), _ptr(out["do"]), _ptr(out["dbias"]), _ptr(out["dC0"]),
                               _ptr(out["dn0"]), _ptr(ws), wsb, _stream(dev))
    _check(rc, "mlstm_chunkwise_bwd")
    return out


def retention_chunkwise_bwd(q, k, v, dout, gamma=None, S0=None, chunk=64, state_grad=True, workspace=None,
                            dS_T=None):
    """retention_chunkwise_bwd: gradients of sum(dout * out) for out =
    retention_chunkwise_fwd(q, k, v, gamma, S0); dS_T [B,H,dk,dv] fp32 or
    None: gradient arriving at the final state.  Returns a dict with dq, dk,
    dv and, with state_grad, dS0 [B,H,dk,dv] fp32."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise TypeError("unsupported dtype %s" % dt)
    _need(q, "q", (B, H, T, dk), dt, dev)
    _need(k, "k", (B, H, T, dk), dt, dev)
    _need(v, "v", (B, H, T, dv), dt, dev)
    _need(dout, "dout", (B, H, T, dv), dt, dev)
    _need(gamma, "gamma", (H,), torch.float32, dev)
    _need(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    _need(dS_T, "dS_T", (B, H, dk, dv), torch.float32, dev)
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dS0=torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev) if state_grad else None)
    L = lib()
    nbytes = L.retention_chunkwise_bwd_workspace_bytes(B, H, T, dk, dv, chunk, _DT[dt])
    if nbytes == 0:
        _check(L.retention_chunkwise_bwd(B, H, T, dk, dv, chunk, _DT[dt], *([None] * 11), None, 0, None),
               "retention_chunkwise_bwd")
    ws, wsb = _workspace(nbytes, dev, workspace)
    rc = L.retention_chunkwise_bwd(B, H, T, dk, dv, chunk, _DT[dt], _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                                   _ptr(S0), _ptr(dout), _ptr(dS_T), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                   _ptr(out["dS0"]), _ptr(ws), wsb, _stream(dev))
    _check(rc, "retention_chunkwise_bwd")
    return out
