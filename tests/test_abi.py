"""C ABI checks that need no GPU: the library loads, exports every function
that include/mlstm.h declares, and rejects invalid arguments with the
documented error codes before touching the GPU (all pointers here are NULL or
bogus host values that the library must never dereference)."""
import ctypes
import os
import re

import pytest

from linear_recurrent_sequence_mlstm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
E_NULL, E_SHAPE, E_DTYPE, E_UNSUPPORTED, E_WORKSPACE = -1, -2, -3, -4, -5


def declared_functions():
    src = open(os.path.join(ROOT, "include", "mlstm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_]+)\s*\(", src)) - {"sizeof"})


def test_header_declares_the_exported_api():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert _lib.abi_version() == 2


BOGUS = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _fwd(B=1, H=2, T=64, dqk=64, dv=64, nb=1, chunk=64, dt=1, ptr=BOGUS, ws=BOGUS, wsb=1 << 30):
    L = _lib.lib()
    p = [ptr] * 6 + [None] * 7
    return L.mlstm_chunkwise_fwd(B, H, T, dqk, dv, nb, chunk, dt, *p, ptr, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), E_SHAPE), (dict(T=0), E_SHAPE), (dict(dqk=-1), E_SHAPE),
    (dict(nb=3), E_SHAPE), (dict(dt=7), E_DTYPE), (dict(chunk=48), E_SHAPE),
    (dict(dqk=96), E_UNSUPPORTED), (dict(dv=96), E_UNSUPPORTED), (dict(nb=4), E_UNSUPPORTED),
    (dict(ptr=None), E_NULL), (dict(ws=None), E_WORKSPACE), (dict(wsb=16), E_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x1008)), E_WORKSPACE),
])
def test_chunkwise_validation(kw, code):
    assert _fwd(**kw) == code
    assert _lib.last_error() != ""


def test_workspace_query():
    L = _lib.lib()
    n = L.mlstm_chunkwise_workspace_bytes(1, 8, 8192, 256, 512, 1, 64, 1)
    assert n > 0 and n % 256 == 0
    assert L.mlstm_chunkwise_workspace_bytes(1, 8, 8192, 96, 512, 1, 64, 1) == 0
    assert L.retention_chunkwise_workspace_bytes(8, 4, 2048, 64, 64, 64, 1) > 0


def test_norm_mode_validation():
    L = _lib.lib()
    p = [BOGUS] * 6 + [None] * 7
    assert L.mlstm_chunkwise_fwd_ex(1, 2, 64, 64, 64, 1, 64, 1, 7, *p, BOGUS, BOGUS, 1 << 30, None) == E_UNSUPPORTED
    assert L.mlstm_chunkwise_fwd_ex(1, 2, 64, 64, 64, 1, 64, 1, 1, *p[:-1], None, None, BOGUS, 1 << 30,
                                    None) == E_NULL
    P0 = [BOGUS] * 6 + [None] + [BOGUS] * 3
    assert L.mlstm_step_ex(1, 1, 64, 64, 1, 1, 9, *P0, BOGUS, None) == E_UNSUPPORTED
    assert L.mlstm_step_ex(1, 1, 64, 60, 1, 1, 1, *P0, BOGUS, None) == E_UNSUPPORTED
    assert L.mlstm_step_ex(1, 1, 64, 64, 16, 1, 2, *P0, BOGUS, None) == E_UNSUPPORTED  # > 8 blocks
    assert _lib.last_error() != ""


def test_step_validation():
    L = _lib.lib()
    P = [BOGUS] * 6 + [None] + [BOGUS] * 3 + [BOGUS, None]
    P0 = [BOGUS] * 6 + [None] + [BOGUS] * 3
    assert L.mlstm_step(0, 1, 64, 64, 1, 1, *P0, BOGUS, None) == E_SHAPE
    assert L.mlstm_step(1, 1, 64, 64, 1, 5, *P0, BOGUS, None) == E_DTYPE
    assert L.mlstm_step(1, 1, 64, 60, 1, 1, *P0, BOGUS, None) == E_UNSUPPORTED
    for dv in (8, 24, 40, 100, 1000):  # outside the documented d_v rule
        assert L.mlstm_step(1, 1, 64, dv, 1, 1, *P0, BOGUS, None) == E_UNSUPPORTED, dv
    assert L.mlstm_step(1, 1, 64, 64, 3, 1, *P0, BOGUS, None) == E_SHAPE
    assert L.mlstm_step(1, 1, 64, 64, 1, 1, *([None] * 10), BOGUS, None) == E_NULL


def test_retention_step_validation():
    L = _lib.lib()
    assert L.retention_step(0, 1, 64, 64, 1, BOGUS, BOGUS, BOGUS, None, BOGUS, BOGUS, None) == E_SHAPE
    assert L.retention_step(1, 1, 64, 64, 9, BOGUS, BOGUS, BOGUS, None, BOGUS, BOGUS, None) == E_DTYPE
    for dv in (8, 24, 100):  # d_v must be a multiple of 16
        assert L.retention_step(1, 1, 64, dv, 1, BOGUS, BOGUS, BOGUS, None, BOGUS, BOGUS, None) == E_UNSUPPORTED
    assert L.retention_step(1, 1, 64, 64, 1, BOGUS, None, BOGUS, None, BOGUS, BOGUS, None) == E_NULL
    assert L.retention_step(1, 1, 64, 64, 1, BOGUS, BOGUS, BOGUS, None, None, BOGUS, None) == E_NULL
    assert _lib.last_error() != ""


def test_retention_groupnorm_validation():
    L = _lib.lib()
    f = ctypes.c_float
    args = lambda dv=64, eps=1e-5, q=BOGUS: [1, 1, 10, 64, dv, 64, 1, q, BOGUS, BOGUS, None, None, None,
                                            None, None, f(eps), BOGUS, BOGUS, 1 << 30, None]
    assert L.retention_chunkwise_groupnorm_fwd(*args(dv=96)) == E_UNSUPPORTED  # d_v a multiple of 64 at d_k 64
    assert L.retention_chunkwise_groupnorm_fwd(*args(eps=0.0)) == E_SHAPE
    assert L.retention_chunkwise_groupnorm_fwd(*args(q=None)) == E_NULL
    assert _lib.last_error() != ""
    # heads wider than one work-group need room for their fp32 rows: the
    # workspace grows by exactly B*H*T*d_v*4 bytes (256-aligned), and a call
    # with only the plain retention workspace is rejected before any launch
    plain = L.retention_chunkwise_workspace_bytes(2, 3, 100, 64, 256, 64, 1)
    gn = L.retention_chunkwise_groupnorm_workspace_bytes(2, 3, 100, 64, 256, 64, 1)
    assert plain > 0 and gn == plain + ((2 * 3 * 100 * 256 * 4 + 255) // 256) * 256
    assert L.retention_chunkwise_groupnorm_workspace_bytes(2, 3, 100, 64, 64, 64, 1) == \
        L.retention_chunkwise_workspace_bytes(2, 3, 100, 64, 64, 64, 1)
    assert L.retention_chunkwise_groupnorm_workspace_bytes(2, 3, 100, 64, 96, 64, 1) == 0
    wide = [2, 3, 100, 64, 256, 64, 1, BOGUS, BOGUS, BOGUS, None, None, None, None, None, f(1e-5), BOGUS]
    assert L.retention_chunkwise_groupnorm_fwd(*wide, BOGUS, plain, None) == E_WORKSPACE


def test_retention_validation():
    L = _lib.lib()
    p = [BOGUS] * 3 + [None] * 3
    assert L.retention_chunkwise_fwd(1, 1, 10, 256, 64, 64, 1, *p, BOGUS, BOGUS, 1 << 30, None) == E_UNSUPPORTED
    assert L.retention_chunkwise_fwd(1, 1, 10, 64, 64, 64, 1, None, BOGUS, BOGUS, None, None, None,
                                     BOGUS, BOGUS, 1 << 30, None) == E_NULL


@pytest.mark.parametrize("dt,T,d", [(0, 1 << 24, 64), (1, 1 << 24, 64), (1, 1 << 22, 512), (0, (1 << 23) + 5, 64)])
def test_slice_bytes_limit(dt, T, d):
    """One (batch, head) of a tensor is addressed with 32-bit byte offsets: a
    slice of 2^31 bytes or more is rejected (forward, workspace queries and
    backward) before anything runs, instead of wrapping."""
    L = _lib.lib()
    assert _fwd(T=T, dqk=64, dv=d, dt=dt) == E_SHAPE
    assert "2^31" in _lib.last_error()
    assert L.mlstm_chunkwise_workspace_bytes(1, 2, T, 64, d, 1, 64, dt) == 0
    assert L.mlstm_chunkwise_bwd_workspace_bytes(1, 2, T, 64, d, 1, 64, dt) == 0
    assert L.retention_chunkwise_workspace_bytes(1, 2, T, 64, d, 64, dt) == 0
    # just below the limit the same shape family plans normally
    Tok = ((1 << 31) // (d * (2 if dt else 4))) - 64
    assert L.mlstm_chunkwise_workspace_bytes(1, 2, Tok, 64, d, 1, 64, dt) > 0


def test_workspace_argument_checks():
    """A caller's workspace must be a contiguous tensor on the call's device;
    its size counts in bytes whatever its dtype (no GPU needed: the checks
    raise before anything is allocated)."""
    import torch
    dev = torch.device("cuda:0")
    with pytest.raises(ValueError, match="workspace is on"):
        _lib._workspace(1024, dev, torch.empty(4096, dtype=torch.uint8))
    with pytest.raises(TypeError):
        _lib._workspace(1024, dev, object())
    cpu = torch.device("cpu")
    ws, n = _lib._workspace(1024, cpu, torch.empty(512, dtype=torch.float32))
    assert n == 2048 and ws.dtype == torch.float32
    with pytest.raises(ValueError, match="contiguous"):
        _lib._workspace(16, cpu, torch.empty(64, 2)[:, 0])


def test_noalloc_rejects_beyond_its_scratch():
    """The no-allocation forward holds a fixed scratch array: a call that
    needs more is rejected before anything runs (no GPU needed), and invalid
    arguments get the same codes as the workspace entry point."""
    L = _lib.lib()
    cap = L.mlstm_noalloc_scratch_bytes()
    assert cap == 64 << 20
    p = [BOGUS] * 6 + [None] * 7
    need = L.mlstm_chunkwise_workspace_bytes(4, 8, 8192, 256, 512, 1, 64, 1)
    assert need > cap
    assert L.mlstm_chunkwise_fwd_noalloc(4, 8, 8192, 256, 512, 1, 64, 1, 0, *p, BOGUS, None) == E_WORKSPACE
    assert "scratch" in _lib.last_error()
    assert L.mlstm_chunkwise_workspace_bytes(1, 8, 8192, 256, 512, 1, 64, 1) <= cap  # the 7B prefill fits
    assert L.mlstm_chunkwise_fwd_noalloc(1, 2, 64, 96, 64, 1, 64, 1, 0, *p, BOGUS, None) == E_UNSUPPORTED
    assert L.mlstm_chunkwise_fwd_noalloc(1, 2, 64, 64, 64, 1, 64, 1, 0, *p, None, None) == E_NULL
    assert L.mlstm_chunkwise_fwd_noalloc(1, 2, 64, 64, 64, 1, 64, 1, 9, *p, BOGUS, None) == E_UNSUPPORTED


def test_binding_workspace_checks():
    """A caller's workspace is used as given or rejected, never replaced: too
    small, on another device, or not contiguous raises (host-side, no GPU)."""
    import torch
    from linear_recurrent_sequence_mlstm_amd._lib import _workspace
    cpu = torch.device("cpu")
    ws = torch.empty(1000, dtype=torch.uint8)
    got, n = _workspace(1000, cpu, ws)
    assert got is ws and n == 1000
    got, n = _workspace(3000, cpu, torch.empty(1000, dtype=torch.float32))  # any dtype, counted in bytes
    assert n == 4000
    with pytest.raises(ValueError):
        _workspace(1001, cpu, ws)
    with pytest.raises(ValueError):
        _workspace(10, cpu, torch.empty(40, dtype=torch.uint8)[::2])
    with pytest.raises(TypeError):
        _workspace(10, cpu, bytearray(100))
    fresh, n = _workspace(10, cpu, None)
    assert n >= 256
