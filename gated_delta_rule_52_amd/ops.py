"""Torch-facing wrappers of the KDA C ABI.

torch supplies device memory and the current HIP stream; every step of the
operator runs in libkda.so.  Shapes and dtypes follow include/kda.h.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import KdaError  # noqa: F401  (re-exported)

_DT = {torch.bfloat16: _lib.KDA_DTYPE_BF16, torch.float32: _lib.KDA_DTYPE_FP32}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, shape, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _flags(qk_l2norm: bool, gate_logits: bool, scalar_gate: bool = False) -> int:
    return ((_lib.KDA_FLAG_QK_L2NORM if qk_l2norm else 0) | (_lib.KDA_FLAG_GATE_SOFTPLUS if gate_logits else 0)
            | (_lib.KDA_FLAG_SCALAR_GATE if scalar_gate else 0))


def _fill_chunk_args(q, k, v, g, beta, initial_state, final_state, o, cu_seqlens, scale,
                     chunk_size, workspace=None, workspace_bytes=0, flags=0, gate_scale=1.0):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    a = _lib.ChunkFwdArgs()
    a.q, a.k, a.v, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    a.initial_state, a.final_state, a.o = _ptr(initial_state), _ptr(final_state), _ptr(o)
    a.cu_seqlens = _ptr(cu_seqlens)
    a.B, a.T, a.H, a.dk, a.dv, a.num_seqs = B, T, H, dk, dv, N
    a.scale = float(scale)
    a.in_dtype = _DT[q.dtype]
    a.out_dtype = _DT[o.dtype]
    a.chunk_size = int(chunk_size)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = int(workspace_bytes)
    a.stream = _stream(q.device)
    a.flags = int(flags)
    a.gate_scale = float(gate_scale)
    return a


def chunk_fwd_workspace_bytes(q, v, cu_seqlens=None, chunk_size: int = 64) -> int:
    B, T, H, dk = q.shape
    a = _lib.ChunkFwdArgs()
    a.B, a.T, a.H, a.dk, a.dv = B, T, H, dk, v.shape[-1]
    a.num_seqs = B if cu_seqlens is None else cu_seqlens.numel() - 1
    a.cu_seqlens = _ptr(cu_seqlens)
    a.scale, a.in_dtype, a.out_dtype, a.chunk_size = 1.0, _DT[q.dtype], _DT[q.dtype], chunk_size
    n = _lib.chunk_workspace_raw(a)
    if n == 2 ** 64 - 1:
        _lib.check(_lib.STATUS_CODE["KDA_ERR_BAD_SHAPE"])
    return int(n)


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
              beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, scale: float = 1.0,
              chunk_size: int = 64, out_dtype: Optional[torch.dtype] = None,
              output_final_state: bool = True, final_state: Optional[torch.Tensor] = None,
              o: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
              qk_l2norm: bool = False, gate_logits: bool = False, gate_scale: float = 1.0,
              scalar_gate: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise KDA prefill.  Returns (o [B,T,H,dv], final_state [N,H,dk,dv] or None).

    q, k: [B,T,H,dk] (bf16 or fp32); v: [B,T,H,dv]; g: [B,T,H,dk] fp32 (log
    decay); beta: [B,T,H]; initial_state: [N,H,dk,dv] fp32 or None;
    cu_seqlens: int32 [N+1] device tensor for packed variable-length input
    (B == 1).  ``final_state`` may be given (it may be ``initial_state`` for an
    in-place update); otherwise one is allocated when ``output_final_state``.

    Input transforms done inside the kernels: ``qk_l2norm`` divides each
    token's q and k by its L2 norm (plus 1e-6 under the root); with
    ``gate_logits`` g holds logits z and the log-gate is
    -gate_scale * softplus(z).  ``scalar_gate``: g is [B,T,H], one gate per token
    and head for every key channel (Gated DeltaNet).
    """
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported input dtype {dt}")
    _need(q, "q", (B, T, H, dk), dt)
    _need(k, "k", (B, T, H, dk), dt)
    _need(v, "v", (B, T, H, dv), dt)
    _need(g, "g", (B, T, H) if scalar_gate else (B, T, H, dk), torch.float32)
    _need(beta, "beta", (B, T, H), dt)
    N = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32)
        N = cu_seqlens.numel() - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", (N, H, dk, dv), torch.float32)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    elif final_state is not None:
        _need(final_state, "final_state", (N, H, dk, dv), torch.float32)
    od = out_dtype or dt
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=od, device=q.device)
    else:
        _need(o, "o", (B, T, H, dv), od)
    ws = chunk_fwd_workspace_bytes(q, v, cu_seqlens, chunk_size)
    if ws > 0 and (workspace is None or workspace.numel() * workspace.element_size() < ws):
        workspace = torch.empty(ws, dtype=torch.uint8, device=q.device)
    a = _fill_chunk_args(q, k, v, g, beta, initial_state, final_state, o, cu_seqlens, scale,
                         chunk_size, workspace, ws if ws > 0 else 0, _flags(qk_l2norm, gate_logits, scalar_gate),
                         gate_scale)
    _lib.check(_lib.chunk_fwd_raw(a))
    return o, final_state


def chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                      beta: torch.Tensor, o: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                      final_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
                      scale: float = 1.0, chunk_size: int = 64, qk_l2norm: bool = False,
                      gate_logits: bool = False, gate_scale: float = 1.0,
                      scalar_gate: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``chunk_fwd`` through kda_chunk_fwd_noalloc: the caller passes every
    output (o, and final_state when wanted), and the library's built-in
    scratch replaces the workspace, so nothing is allocated on this path.
    Problems whose workspace exceeds the built-in scratch raise KdaError
    (KDA_ERR_WORKSPACE_TOO_SMALL).  Returns (o, final_state)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported input dtype {dt}")
    _need(q, "q", (B, T, H, dk), dt)
    _need(k, "k", (B, T, H, dk), dt)
    _need(v, "v", (B, T, H, dv), dt)
    _need(g, "g", (B, T, H) if scalar_gate else (B, T, H, dk), torch.float32)
    _need(beta, "beta", (B, T, H), dt)
    N = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32)
        N = cu_seqlens.numel() - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", (N, H, dk, dv), torch.float32)
    if final_state is not None:
        _need(final_state, "final_state", (N, H, dk, dv), torch.float32)
    if o.dtype not in _DT:
        raise ValueError(f"unsupported output dtype {o.dtype}")
    _need(o, "o", (B, T, H, dv), o.dtype)
    a = _fill_chunk_args(q, k, v, g, beta, initial_state, final_state, o, cu_seqlens, scale,
                         chunk_size, None, 0, _flags(qk_l2norm, gate_logits, scalar_gate), gate_scale)
    _lib.check(_lib.chunk_fwd_noalloc_raw(a))
    return o, final_state


def recurrent_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                  cu_seqlens: Optional[torch.Tensor] = None, scale: float = 1.0,
                  out_dtype: Optional[torch.dtype] = None, output_final_state: bool = True,
                  final_state: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None,
                  qk_l2norm: bool = False, gate_logits: bool = False, gate_scale: float = 1.0,
                  scalar_gate: bool = False, token_by_token: bool = False,
                  workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Fused recurrent forward for short segments: the same arguments, shapes,
    input transforms and results as ``chunk_fwd`` (no chunk size).  Calls with
    more than 16 tokens per sequence on average are handed a chunk workspace,
    with which kda_recurrent_fwd runs the faster chunkwise path; with
    ``token_by_token`` no workspace is passed and the token kernel always runs.
    Returns (o, final_state)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported input dtype {dt}")
    _need(q, "q", (B, T, H, dk), dt)
    _need(k, "k", (B, T, H, dk), dt)
    _need(v, "v", (B, T, H, dv), dt)
    _need(g, "g", (B, T, H) if scalar_gate else (B, T, H, dk), torch.float32)
    _need(beta, "beta", (B, T, H), dt)
    N = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32)
        N = cu_seqlens.numel() - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", (N, H, dk, dv), torch.float32)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    elif final_state is not None:
        _need(final_state, "final_state", (N, H, dk, dv), torch.float32)
    od = out_dtype or dt
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=od, device=q.device)
    else:
        _need(o, "o", (B, T, H, dv), od)
    ws = 0
    if not token_by_token and B * T > 16 * N:
        ws = chunk_fwd_workspace_bytes(q, v, cu_seqlens, 64)
        if ws > 0 and (workspace is None or workspace.numel() * workspace.element_size() < ws):
            workspace = torch.empty(ws, dtype=torch.uint8, device=q.device)
    a = _fill_chunk_args(q, k, v, g, beta, initial_state, final_state, o, cu_seqlens, scale, 64,
                         workspace if ws > 0 else None, ws,
                         flags=_flags(qk_l2norm, gate_logits, scalar_gate), gate_scale=gate_scale)
    _lib.check(_lib.recurrent_fwd_raw(a))
    return o, final_state


def recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                   beta: torch.Tensor, state: Optional[torch.Tensor],
                   final_state: Optional[torch.Tensor] = None, scale: float = 1.0,
                   out_dtype: Optional[torch.dtype] = None,
                   o: Optional[torch.Tensor] = None, qk_l2norm: bool = False,
                   gate_logits: bool = False, gate_scale: float = 1.0,
                   scalar_gate: bool = False) -> torch.Tensor:
    """One decode step for N sequences.  q, k, g: [N,H,dk]; v: [N,H,dv];
    beta: [N,H]; state: [N,H,dk,dv] fp32 (or None for zeros).  The new state
    is written to ``final_state`` (default: ``state`` itself, in place).
    Input transforms as in ``chunk_fwd``.  Returns o [N,H,dv]."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported input dtype {dt}")
    _need(q, "q", (N, H, dk), dt)
    _need(k, "k", (N, H, dk), dt)
    _need(v, "v", (N, H, dv), dt)
    _need(g, "g", (N, H) if scalar_gate else (N, H, dk), torch.float32)
    _need(beta, "beta", (N, H), dt)
    if state is not None:
        _need(state, "state", (N, H, dk, dv), torch.float32)
    if final_state is None:
        if state is None:
            raise ValueError("final_state is required when state is None")
        final_state = state
    _need(final_state, "final_state", (N, H, dk, dv), torch.float32)
    od = out_dtype or dt
    if o is None:
        o = torch.empty((N, H, dv), dtype=od, device=q.device)
    a = _lib.RecurrentStepArgs()
    a.q, a.k, a.v, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    a.initial_state, a.final_state, a.o = _ptr(state), _ptr(final_state), _ptr(o)
    a.N, a.H, a.dk, a.dv = N, H, dk, dv
    a.scale = float(scale)
    a.in_dtype = _DT[dt]
    a.out_dtype = _DT[od]
    a.stream = _stream(q.device)
    a.flags = _flags(qk_l2norm, gate_logits, scalar_gate)
    a.gate_scale = float(gate_scale)
    _lib.check(_lib.recurrent_step_raw(a))
    return o


def _bwd_args(q, v, cu_seqlens, scale, scalar_gate=False, qk_l2norm=False, gate_logits=False, gate_scale=1.0):
    B, T, H, dk = q.shape
    a = _lib.RecurrentBwdArgs()
    a.flags = _flags(qk_l2norm, gate_logits, scalar_gate)
    a.gate_scale = float(gate_scale)
    a.B, a.T, a.H, a.dk, a.dv = B, T, H, dk, v.shape[-1]
    a.num_seqs = B if cu_seqlens is None else cu_seqlens.numel() - 1
    a.cu_seqlens = _ptr(cu_seqlens)
    a.scale = float(scale)
    a.in_dtype = _DT[q.dtype]
    return a


def recurrent_bwd_workspace_bytes(q, v, cu_seqlens=None, scalar_gate=False, qk_l2norm=False,
                                  gate_logits=False) -> int:
    n = _lib.recurrent_bwd_workspace_raw(_bwd_args(q, v, cu_seqlens, 1.0, scalar_gate, qk_l2norm, gate_logits))
    if n == 2 ** 64 - 1:
        _lib.check(_lib.STATUS_CODE["KDA_ERR_BAD_SHAPE"])
    return int(n)


def chunk_bwd_workspace_bytes(q, v, cu_seqlens=None) -> int:
    n = _lib.chunk_bwd_workspace_raw(_bwd_args(q, v, cu_seqlens, 1.0, False, False, False))
    if n == 2 ** 64 - 1:
        _lib.check(_lib.STATUS_CODE["KDA_ERR_UNSUPPORTED"])
    return int(n)


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
              beta: torch.Tensor, grad_o: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
              grad_final_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, scale: float = 1.0,
              output_grad_initial_state: bool = True, grad_initial_state: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None):
    """The gradients of ``recurrent_bwd`` by the chunk path (bf16 inputs,
    dk = dv = 128, no input transforms); same arguments and result."""
    return _backward(q, k, v, g, beta, grad_o, initial_state, grad_final_state, cu_seqlens, scale,
                     output_grad_initial_state, grad_initial_state, workspace, out, False, False, False, 1.0,
                     chunk=True)


def recurrent_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  beta: torch.Tensor, grad_o: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                  grad_final_state: Optional[torch.Tensor] = None,
                  cu_seqlens: Optional[torch.Tensor] = None, scale: float = 1.0,
                  output_grad_initial_state: bool = True, grad_initial_state: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None,
                  scalar_gate: bool = False, qk_l2norm: bool = False, gate_logits: bool = False,
                  gate_scale: float = 1.0):
    """Gradients of the recurrence for the output
    gradient ``grad_o`` [B,T,H,dv] (dtype of q) and the optional final-state
    gradient [N,H,dk,dv] fp32.  Inputs as in ``chunk_fwd``.  Returns a dict of
    fp32 tensors: dq, dk, dg [B,T,H,dk], dv [B,T,H,dv], dbeta [B,T,H] and dh0
    [N,H,dk,dv] (None unless ``output_grad_initial_state`` or
    ``grad_initial_state`` is given; the latter may be ``initial_state`` or
    ``grad_final_state`` for an in-place result).  ``out`` may supply the
    token gradients (a dict with dq, dk, dv, dg, dbeta), written in place.
    ``scalar_gate``: g (and dg) are [B,T,H], one gate per token and head.
    ``qk_l2norm``, ``gate_logits``, ``gate_scale``: the forward's input
    transforms; dq, dk and dg are then gradients of the raw q, k and logits."""
    return _backward(q, k, v, g, beta, grad_o, initial_state, grad_final_state, cu_seqlens, scale,
                     output_grad_initial_state, grad_initial_state, workspace, out, scalar_gate, qk_l2norm,
                     gate_logits, gate_scale, chunk=False)


def _backward(q, k, v, g, beta, grad_o, initial_state, grad_final_state, cu_seqlens, scale,
              output_grad_initial_state, grad_initial_state, workspace, out, scalar_gate, qk_l2norm,
              gate_logits, gate_scale, chunk):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported input dtype {dt}")
    _need(q, "q", (B, T, H, dk), dt)
    _need(k, "k", (B, T, H, dk), dt)
    _need(v, "v", (B, T, H, dv), dt)
    _need(g, "g", (B, T, H) if scalar_gate else (B, T, H, dk), torch.float32)
    _need(beta, "beta", (B, T, H), dt)
    _need(grad_o, "grad_o", (B, T, H, dv), dt)
    N = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32)
        N = cu_seqlens.numel() - 1
    for name, t in (("initial_state", initial_state), ("grad_final_state", grad_final_state)):
        if t is not None:
            _need(t, name, (N, H, dk, dv), torch.float32)
    if grad_initial_state is None and output_grad_initial_state:
        grad_initial_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    elif grad_initial_state is not None:
        _need(grad_initial_state, "grad_initial_state", (N, H, dk, dv), torch.float32)
    f32 = dict(dtype=torch.float32, device=q.device)
    shapes = dict(dq=(B, T, H, dk), dk=(B, T, H, dk), dv=(B, T, H, dv),
                  dg=(B, T, H) if scalar_gate else (B, T, H, dk), dbeta=(B, T, H))
    if out is None:
        out = {n: torch.empty(sh, **f32) for n, sh in shapes.items()}
    else:
        out = {n: out[n] for n in shapes}
        for n, sh in shapes.items():
            _need(out[n], n, sh, torch.float32)
    out["dh0"] = grad_initial_state
    ws = (chunk_bwd_workspace_bytes(q, v, cu_seqlens) if chunk else
          recurrent_bwd_workspace_bytes(q, v, cu_seqlens, scalar_gate, qk_l2norm, gate_logits))
    if ws > 0 and (workspace is None or workspace.numel() * workspace.element_size() < ws):
        workspace = torch.empty(ws, dtype=torch.uint8, device=q.device)
    a = _bwd_args(q, v, cu_seqlens, scale, scalar_gate, qk_l2norm, gate_logits, gate_scale)
    a.q, a.k, a.v, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    a.initial_state, a.grad_o, a.grad_final_state = _ptr(initial_state), _ptr(grad_o), _ptr(grad_final_state)
    a.grad_q, a.grad_k, a.grad_v = _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"])
    a.grad_g, a.grad_beta, a.grad_initial_state = _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(grad_initial_state)
    a.workspace = _ptr(workspace) if ws > 0 else None
    a.workspace_bytes = ws
    a.stream = _stream(q.device)
    _lib.check(_lib.chunk_bwd_raw(a) if chunk else _lib.recurrent_bwd_raw(a))
    return out


def dplr_recurrent_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                       a: torch.Tensor, b: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                       cu_seqlens: Optional[torch.Tensor] = None, scale: float = 1.0,
                       out_dtype: Optional[torch.dtype] = None, output_final_state: bool = True,
                       final_state: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None):
    """The general DPLR recurrence S_t = (Diag(e^g_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,
    o_t = scale S_t^T q_t, token by token.  q, k, a, b: [B,T,H,dk] (bf16 or fp32); v: [B,T,H,dv];
    g: [B,T,H,dk] fp32; states and cu_seqlens as in ``chunk_fwd``.  Returns (o, final_state)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported input dtype {dt}")
    for name, t in (("q", q), ("k", k), ("a", a), ("b", b)):
        _need(t, name, (B, T, H, dk), dt)
    _need(v, "v", (B, T, H, dv), dt)
    _need(g, "g", (B, T, H, dk), torch.float32)
    N = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32)
        N = cu_seqlens.numel() - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", (N, H, dk, dv), torch.float32)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    elif final_state is not None:
        _need(final_state, "final_state", (N, H, dk, dv), torch.float32)
    od = out_dtype or dt
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=od, device=q.device)
    else:
        _need(o, "o", (B, T, H, dv), od)
    x = _lib.DplrArgs()
    x.q, x.k, x.v, x.g, x.a, x.b = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(a), _ptr(b)
    x.initial_state, x.final_state, x.o = _ptr(initial_state), _ptr(final_state), _ptr(o)
    x.cu_seqlens = _ptr(cu_seqlens)
    x.B, x.T, x.H, x.dk, x.dv, x.num_seqs = B, T, H, dk, dv, N
    x.scale = float(scale)
    x.in_dtype, x.out_dtype = _DT[dt], _DT[od]
    x.stream = _stream(q.device)
    _lib.check(_lib.dplr_fwd_raw(x))
    return o, final_state


def dplr_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                   a: torch.Tensor, b: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                   cu_seqlens: Optional[torch.Tensor] = None, scale: float = 1.0,
                   out_dtype: Optional[torch.dtype] = None, output_final_state: bool = True,
                   final_state: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None):
    """The general DPLR recurrence of ``dplr_recurrent_fwd`` in chunkwise form (kda_dplr_chunk_fwd):
    same arguments and results, plus an optional caller workspace.  Returns (o, final_state)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported input dtype {dt}")
    for name, t in (("q", q), ("k", k), ("a", a), ("b", b)):
        _need(t, name, (B, T, H, dk), dt)
    _need(v, "v", (B, T, H, dv), dt)
    _need(g, "g", (B, T, H, dk), torch.float32)
    N = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32)
        N = cu_seqlens.numel() - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", (N, H, dk, dv), torch.float32)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    elif final_state is not None:
        _need(final_state, "final_state", (N, H, dk, dv), torch.float32)
    od = out_dtype or dt
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=od, device=q.device)
    else:
        _need(o, "o", (B, T, H, dv), od)
    x = _lib.DplrChunkArgs()
    x.q, x.k, x.v, x.g, x.a, x.b = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(a), _ptr(b)
    x.initial_state, x.final_state, x.o = _ptr(initial_state), _ptr(final_state), _ptr(o)
    x.cu_seqlens = _ptr(cu_seqlens)
    x.B, x.T, x.H, x.dk, x.dv, x.num_seqs = B, T, H, dk, dv, N
    x.scale = float(scale)
    x.in_dtype, x.out_dtype = _DT[dt], _DT[od]
    ws = _lib.dplr_chunk_workspace_raw(x)
    if ws == 2 ** 64 - 1:
        _lib.check(_lib.STATUS_CODE["KDA_ERR_BAD_SHAPE"])
    if ws > 0 and (workspace is None or workspace.numel() * workspace.element_size() < ws):
        workspace = torch.empty(ws, dtype=torch.uint8, device=q.device)
    x.workspace = _ptr(workspace) if ws > 0 else None
    x.workspace_bytes = int(ws)
    x.stream = _stream(q.device)
    _lib.check(_lib.dplr_chunk_fwd_raw(x))
    return o, final_state
