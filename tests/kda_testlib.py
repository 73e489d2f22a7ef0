"""Helpers shared by the GPU parity tests: device upload, the parity gate, and
the oracle call on selected heads.

The gate (class Gate) works on slices: one slice is a 2-D array [rows, cols]
for one (sequence, head), either token rows of an output ([tokens, dv]) or key
rows of a state ([dk, dv]).  Two quantities are gated, both at the same
tolerance:

* slice:  ||gpu - ref||_F / ||ref||_F;
* row:    ||gpu_r - ref_r|| / max(||ref_r||, ||ref||_F / sqrt(rows)) for every
          row r, so that one wrong token (or key row) cannot hide in a long
          slice.  The floor is the slice's RMS row norm: a row whose reference
          is much smaller than its neighbours is judged against the typical
          row, not against its own near-zero norm.

Reported beside them, not gated: max |gpu - ref|, the rms of gpu - ref, and
that rms relative to the rms of ref.
"""
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


class Gate:
    """Parity metrics of one quantity (o, the final state, a gradient) over
    (sequence, head) slices; see the module docstring."""

    def __init__(self, name, tol):
        self.name, self.tol = name, tol
        self.slice_err = 0.0
        self.row_err = 0.0
        self.max_abs = 0.0
        self.sq, self.ref_sq, self.count, self.slices = 0.0, 0.0, 0, 0

    def add(self, gpu, ref):
        """One slice; a 1-D slice is a column of one-element rows."""
        gpu = np.asarray(gpu, np.float64)
        ref = np.asarray(ref, np.float64)
        if gpu.ndim == 1:
            gpu, ref = gpu[:, None], ref[:, None]
        gpu = gpu.reshape(gpu.shape[0], -1)
        ref = ref.reshape(ref.shape[0], -1)
        assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
        self.slices += 1
        if gpu.size == 0:
            return
        if not np.isfinite(gpu).all():  # a non-finite result is an infinite error
            self.slice_err = self.row_err = self.max_abs = float("inf")
            return
        diff = gpu - ref
        nref = np.linalg.norm(ref)
        self.slice_err = max(self.slice_err, np.linalg.norm(diff) / max(nref, 1e-30))
        floor = max(nref / np.sqrt(ref.shape[0]), 1e-30)
        rows = np.linalg.norm(diff, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), floor)
        self.row_err = max(self.row_err, float(rows.max()))
        self.max_abs = max(self.max_abs, float(np.abs(diff).max()))
        self.sq += float((diff * diff).sum())
        self.ref_sq += float((ref * ref).sum())
        self.count += diff.size

    @property
    def worst(self):
        return max(self.slice_err, self.row_err)

    def report(self):
        rms = np.sqrt(self.sq / max(self.count, 1))
        rms_ref = np.sqrt(self.ref_sq / max(self.count, 1))
        return (f"{self.name}: slice {self.slice_err:.3e} row {self.row_err:.3e} | max-abs {self.max_abs:.3e} "
                f"rms {rms:.3e} (rms/rms_ref {rms / max(rms_ref, 1e-30):.3e}) over {self.slices} slices")

    def ok(self):
        return self.slice_err <= self.tol and self.row_err <= self.tol


def gate_all(gates):
    """Print every gate and fail if any exceeds its tolerance."""
    for g in gates:
        say("  " + g.report() + f" (tol {g.tol:g})")
    bad = [g.report() for g in gates if not g.ok()]
    assert not bad, bad


def prefill_gates(o_gpu, hT_gpu, o_ref, hT_ref, x, heads, tol):
    """Gates for o ([B,T,H,dv], all heads on the GPU side; the refs hold the
    listed heads only) and the final state, one slice per (sequence, head)."""
    o_gpu = np.asarray(o_gpu).reshape(-1, o_gpu.shape[2], o_gpu.shape[3])
    o_ref = np.asarray(o_ref).reshape(-1, o_ref.shape[2], o_ref.shape[3])
    go, gs = Gate("o", tol), Gate("state", tol)
    for n, (a, b) in enumerate(x.seq_bounds()):
        for j, h in enumerate(heads):
            if b > a:
                go.add(o_gpu[a:b, h], o_ref[a:b, j])
            if hT_gpu is not None:
                gs.add(hT_gpu[n, h], hT_ref[n, j])
    return go, gs


def check_prefill_outputs(o_gpu, hT_gpu, o_ref, hT_ref, x, heads, tol):
    """Gate o and the final state of a prefill problem; returns the gates."""
    go, gs = prefill_gates(o_gpu, hT_gpu, o_ref, hT_ref, x, heads, tol)
    gate_all([go, gs] if hT_gpu is not None else [go])
    return go, gs


def oracle_forward(x, heads, scale=1.0):
    return oracle.forward(x.q, x.k, x.v, x.g, x.beta, h0=None if x.h0 is None else x.h0.astype(np.float64),
                          cu_seqlens=x.cu_seqlens, scale=scale, heads=heads)
