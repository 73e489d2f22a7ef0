"""fp64 CPU oracle for the Kimi Delta Attention (KDA) operator.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  Nothing here is used by,
or uses, the HIP path.

* ``forward``: the token-by-token fp64 recurrence (C, OpenMP), see
  ``kda_oracle.c`` for the definition it follows.
* ``backward``: its gradients by reverse-mode differentiation (C, fp64).
* ``reference``: independent numpy special cases and the fp64 chunked form.

Parity status: every function here is pinned by ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        i64, dp, fp = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_float)
        lib.kda_oracle_forward.restype = ctypes.c_int
        lib.kda_oracle_forward.argtypes = [
            i64, ctypes.POINTER(ctypes.c_int64), i64, i64, i64,
            fp, fp, fp, fp, fp, dp, ctypes.c_double,
            ctypes.POINTER(ctypes.c_int32), i64, dp, dp, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int]
        lib.kda_oracle_backward.restype = ctypes.c_int
        lib.kda_oracle_backward.argtypes = [
            i64, ctypes.POINTER(ctypes.c_int64), i64, i64, i64,
            fp, fp, fp, fp, fp, dp, ctypes.c_double, fp, dp,
            dp, dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double]
        lib.kda_oracle_dplr_forward.restype = ctypes.c_int
        lib.kda_oracle_dplr_forward.argtypes = [
            i64, ctypes.POINTER(ctypes.c_int64), i64, i64, i64,
            fp, fp, fp, fp, fp, fp, dp, ctypes.c_double, dp, dp, ctypes.c_int]
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a, t):
    return a.ctypes.data_as(ctypes.POINTER(t)) if a is not None else None


def forward(q, k, v, g, beta, h0=None, cu_seqlens=None, scale: float = 1.0,
            heads: Optional[Sequence[int]] = None, nthreads: int = 0,
            want_state: bool = True, qk_l2norm: bool = False,
            gate_logits: bool = False, gate_scale: float = 1.0, scalar_gate: bool = False):
    """fp64 token recurrence.

    q, k, g: [B, T, H, dk]; v: [B, T, H, dv]; beta: [B, T, H] (any float
    dtype, taken as float32 exact values); h0: [N, H, dk, dv] or None;
    cu_seqlens: [N+1] offsets into the flattened B*T token axis, or None for
    B fixed-length sequences.  Returns (o [B, T, nh, dv], hT [N, nh, dk, dv])
    in float64 for the requested heads (all heads by default).  h0 is taken
    in float64 so a state can be chained between calls without rounding.

    qk_l2norm: q and k are L2-normalised per token and head first
    (x / sqrt(sum x^2 + 1e-6)).  gate_logits: g holds logits z and the
    log-gate is -gate_scale * softplus(z).  Both in fp64, see kda_oracle.c.
    scalar_gate: g is [B, T, H], one gate per token and head for all key
    channels (Gated DeltaNet).
    """
    lib = _load()
    q, k, v, g, beta = map(_f32, (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    hs = np.arange(H, dtype=np.int32) if heads is None else np.ascontiguousarray(heads, dtype=np.int32)
    nh = len(hs)
    o = np.zeros((B, T, nh, dv), dtype=np.float64)
    hT = np.zeros((N, nh, dk, dv), dtype=np.float64) if want_state else None
    h0a = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
    rc = lib.kda_oracle_forward(
        N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk, dv,
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(g, ctypes.c_float), _ptr(beta, ctypes.c_float), _ptr(h0a, ctypes.c_double),
        float(scale), hs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), nh,
        _ptr(o, ctypes.c_double), _ptr(hT, ctypes.c_double), int(nthreads),
        int(bool(qk_l2norm)), int(bool(gate_logits)), float(gate_scale), int(bool(scalar_gate)))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_forward failed with code {rc}")
    return o, hT


def backward(q, k, v, g, beta, d_o, h0=None, d_final_state=None, cu_seqlens=None,
             scale: float = 1.0, nthreads: int = 0, scalar_gate: bool = False, qk_l2norm: bool = False,
             gate_logits: bool = False, gate_scale: float = 1.0):
    """Gradients of the fp64 recurrence (no input transforms) for output
    gradient d_o [B, T, H, dv] and optional final-state gradient
    [N, H, dk, dv].  Returns a dict of float64 arrays: dq, dk, dg [B, T, H, dk],
    dv [B, T, H, dv], dbeta [B, T, H], dh0 [N, H, dk, dv].  With scalar_gate,
    g and dg are [B, T, H] (Gated DeltaNet's gate).  With the input transforms
    of ``forward`` the gradients are those of the raw q, k and gate logits
    (chain rule through the L2 norm and the softplus gate, kda_oracle.c)."""
    lib = _load()
    q, k, v, g, beta, d_o = map(_f32, (q, k, v, g, beta, d_o))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    cu = np.arange(B + 1, dtype=np.int64) * T if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, np.int64)
    N = len(cu) - 1
    out = dict(dq=np.zeros((B, T, H, dk)), dk=np.zeros((B, T, H, dk)), dv=np.zeros((B, T, H, dv)),
               dg=np.zeros((B, T, H) if scalar_gate else (B, T, H, dk)), dbeta=np.zeros((B, T, H)),
               dh0=np.zeros((N, H, dk, dv)))
    h0a = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
    dhT = None if d_final_state is None else np.ascontiguousarray(d_final_state, dtype=np.float64)
    rc = lib.kda_oracle_backward(
        N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk, dv,
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(g, ctypes.c_float), _ptr(beta, ctypes.c_float), _ptr(h0a, ctypes.c_double),
        float(scale), _ptr(d_o, ctypes.c_float), _ptr(dhT, ctypes.c_double),
        *(_ptr(out[n], ctypes.c_double) for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0")), int(nthreads),
        int(bool(scalar_gate)), int(bool(qk_l2norm)), int(bool(gate_logits)), float(gate_scale))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_backward failed with code {rc}")
    return out


def dplr_forward(q, k, v, g, a, b, h0=None, cu_seqlens=None, scale: float = 1.0, nthreads: int = 0):
    """fp64 general DPLR recurrence S_t = (Diag(e^g_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,
    o_t = scale S_t^T q_t (kda_oracle.c).  q, k, g, a, b: [B, T, H, dk]; v: [B, T, H, dv];
    h0: [N, H, dk, dv] or None.  Returns (o [B, T, H, dv], hT [N, H, dk, dv]) in float64."""
    lib = _load()
    q, k, v, g, a, b = map(_f32, (q, k, v, g, a, b))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    cu = np.arange(B + 1, dtype=np.int64) * T if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, np.int64)
    N = len(cu) - 1
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    hT = np.zeros((N, H, dk, dv), dtype=np.float64)
    h0a = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
    rc = lib.kda_oracle_dplr_forward(
        N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk, dv,
        *(_ptr(x, ctypes.c_float) for x in (q, k, v, g, a, b)), _ptr(h0a, ctypes.c_double), float(scale),
        _ptr(o, ctypes.c_double), _ptr(hT, ctypes.c_double), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_dplr_forward failed with code {rc}")
    return o, hT


def decode_step(q, k, v, g, beta, state, scale: float = 1.0, nthreads: int = 0, **transforms):
    """One recurrent step for N independent sequences.

    q, k, g: [N, H, dk]; v: [N, H, dv]; beta: [N, H]; state: [N, H, dk, dv].
    A decode step is the recurrence over a sequence of length one, so this
    runs ``forward`` with N one-token sequences.  Returns (o [N, H, dv],
    new_state [N, H, dk, dv]) in float64.
    """
    N = q.shape[0]
    cu = np.arange(N + 1, dtype=np.int64)
    o, hT = forward(q[None], k[None], v[None], g[None], beta[None], h0=state,
                    cu_seqlens=cu, scale=scale, nthreads=nthreads, **transforms)
    return o[0], hT
