"""MI355X-native mLSTM matrix-memory recurrence (chunkwise prefill, fused
decode step, block-diagonal variant, RetNet retention, chunkwise backward).

The compute runs in ``libmlstm.so`` (hand-written HIP for gfx950) behind a
C ABI declared in ``include/mlstm.h``; :mod:`._lib` marshals torch tensors to
that ABI.  Import is cheap: the library is loaded on first use and its absence
raises an error (there is no fallback path).
"""

__all__ = ["chunkwise_fwd", "chunkwise_bwd", "step", "retention_chunkwise_fwd", "retention_chunkwise_bwd",
           "chunkwise_workspace_bytes", "abi_version", "library_path"]


def __getattr__(name):
    if name in __all__:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
