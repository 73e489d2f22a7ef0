"""Kimi Delta Attention (KDA) on MI355X (gfx950): chunkwise prefill and
recurrent decode, and the gradients of the recurrence, as hand-written HIP
kernels behind a C ABI (include/kda.h).

The Python layer only marshals arguments: torch tensors supply device memory
and the current HIP stream; every step of the operator runs in libkda.so.
"""
__all__ = ["chunk_fwd", "recurrent_fwd", "recurrent_step", "recurrent_bwd", "KdaError", "chunk_fwd_workspace_bytes",
           "recurrent_bwd_workspace_bytes", "dplr_recurrent_fwd", "chunk_fwd_noalloc",
           "dplr_chunk_fwd", "chunk_bwd", "chunk_bwd_workspace_bytes"]


def __getattr__(name):
    if name in __all__:
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
