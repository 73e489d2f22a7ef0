"""Helpers shared by the GPU parity tests: device upload, the norm-wise
per-(sequence, head) error metric, and the oracle call on selected heads."""
import sys

import numpy as np

import oracle

TOL_BF16 = 2e-3   # bf16 inputs, fp32 accumulation and output
TOL_FP32 = 1e-5   # all-fp32 inputs


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device="cuda").to(dtype)


def in_dtype_of(x):
    import torch
    return torch.bfloat16 if x.in_dtype == "bf16" else torch.float32


def upload(x):
    """Device tensors for a KdaInputs problem."""
    import torch
    dt = in_dtype_of(x)
    d = dict(q=dev(x.q, dt), k=dev(x.k, dt), v=dev(x.v, dt), g=dev(x.g, torch.float32),
             beta=dev(x.beta, dt))
    d["h0"] = None if x.h0 is None else dev(x.h0, torch.float32)
    d["cu"] = None if x.cu_seqlens is None else dev(x.cu_seqlens, torch.int32)
    return d


def slice_errors(o_gpu, hT_gpu, o_ref, hT_ref, x, heads):
    """Max over (sequence, head) slices of ||gpu - ref||_F / ||ref||_F for o and
    the final state; o_gpu is [B,T,H,dv] (all heads) and the refs hold the
    listed heads only."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64).reshape(-1, o_gpu.shape[2], o_gpu.shape[3])
    o_ref = np.asarray(o_ref, dtype=np.float64).reshape(-1, o_ref.shape[2], o_ref.shape[3])
    # a non-finite result is an infinite error (max() would drop a NaN)
    if not np.isfinite(o_gpu).all() or (hT_gpu is not None and not np.isfinite(np.asarray(hT_gpu)).all()):
        return float("inf"), float("inf")
    eo, es = 0.0, 0.0
    for n, (a, b) in enumerate(x.seq_bounds()):
        for j, h in enumerate(heads):
            if b > a:
                r = o_ref[a:b, j]
                eo = max(eo, np.linalg.norm(o_gpu[a:b, h] - r) / max(np.linalg.norm(r), 1e-30))
            if hT_gpu is not None:
                r = hT_ref[n, j]
                es = max(es, np.linalg.norm(np.asarray(hT_gpu[n, h], np.float64) - r) / max(np.linalg.norm(r), 1e-30))
    return eo, es


def oracle_forward(x, heads, scale=1.0):
    return oracle.forward(x.q, x.k, x.v, x.g, x.beta, h0=None if x.h0 is None else x.h0.astype(np.float64),
                          cu_seqlens=x.cu_seqlens, scale=scale, heads=heads)
