"""Seeded synthetic inputs for the KDA operator.

This module only draws random numbers and shapes them into the operator's
input layout. It holds none of the operator's arithmetic, so that both the
HIP path and the fp64 oracle can be fed the very same values.

Distributions follow the Kimi Linear operator setting (per-token,
per-head scalar beta from a sigmoid; per-channel log-gate g with
alpha = exp(g); L2-normalised queries and keys):

* q, k ~ N(0, 1), then L2-normalised per (token, head) in float32;
* v ~ N(0, 1);
* beta = sigmoid(N(0, 1));
* g = -gscale * softplus(N(0, 1))   (gscale = 1, or 0.01 for the
  long-retention workload), softplus(x) = log1p(exp(-|x|)) + max(x, 0);
* optional initial state h0 ~ N(0, 0.02^2) (standard deviation 0.02).

With ``fused=True`` the same draws are returned before the last two steps,
for kernels that apply them themselves: q and k are left unnormalised
(bf16-rounded N(0, 1) draws) and ``g`` holds the gate logits z ~ N(0, 1),
the log-gate being -gscale * softplus(z).  ``transforms()`` names what the
consumer must then apply.

With ``scalar_gate=True`` the gate logits are drawn per token and head only
([B, T, H]): one forget rate for every key channel, Gated DeltaNet's gate.

bf16 inputs are rounded once, round-to-nearest-even, and returned as float32
arrays that hold the exact bf16 values, so converting them to bf16 on the
device is lossless and the oracle sees exactly what the GPU sees.

Draw order for one generator: [sequence lengths], q, k, v, beta-logits,
g-logits, h0.  For the decode workload the state is drawn first, then per
step q, k, v, beta-logits, g-logits; a long decode run cycles through a pool
of such per-step batches.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Iterator, Optional

import numpy as np

__all__ = [
    "KdaInputs", "bf16_round", "l2_normalise", "softplus", "sigmoid",
    "make_prefill", "make_output_grads", "make_dplr", "make_decode_state", "decode_steps", "decode_step_pool", "WORKLOADS",
    "make_workload",
]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    r = (b >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += b                       # wraps only for NaN payloads
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32)


def l2_normalise(x: np.ndarray) -> np.ndarray:
    """Normalise the last axis to unit L2 norm in float32."""
    x = x.astype(np.float32, copy=False)
    n = np.sqrt(np.einsum("...i,...i->...", x, x))[..., None]
    return np.divide(x, n, dtype=np.float32)


def softplus(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32, copy=False)
    return (np.log1p(np.exp(-np.abs(x))) + np.maximum(x, 0)).astype(np.float32)


def sigmoid(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32, copy=False)
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


@dataclass
class KdaInputs:
    """One prefill problem, every array float32 holding exact input values.

    q, k, g: [B, T, H, dk]; v: [B, T, H, dv]; beta: [B, T, H];
    h0: [N, H, dk, dv] or None; cu_seqlens: int32 [N+1] or None (then N = B).
    in_dtype is "bf16" or "fp32": the dtype q, k, v and beta travel in.
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    h0: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]
    in_dtype: str
    name: str = ""
    meta: dict = field(default_factory=dict)
    fused: bool = False  # q, k unnormalised and g = gate logits (see module docstring)
    scalar_gate: bool = False  # g is [B, T, H]: one gate per token and head

    def transforms(self) -> dict:
        """Input forms the consumer handles: the gate layout, and for ``fused``
        inputs the in-kernel L2 norm and the softplus gate with its scale."""
        if not self.fused:
            return dict(qk_l2norm=False, gate_logits=False, gate_scale=1.0, scalar_gate=self.scalar_gate)
        return dict(qk_l2norm=True, gate_logits=True, gate_scale=float(self.meta["gscale"]),
                    scalar_gate=self.scalar_gate)

    @property
    def B(self) -> int:
        return self.q.shape[0]

    @property
    def T(self) -> int:
        return self.q.shape[1]

    @property
    def H(self) -> int:
        return self.q.shape[2]

    @property
    def dk(self) -> int:
        return self.q.shape[3]

    @property
    def dv(self) -> int:
        return self.v.shape[3]

    @property
    def N(self) -> int:
        return self.B if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    def seq_bounds(self):
        """(start, end) token offsets of each sequence in the flattened [B*T] axis."""
        if self.cu_seqlens is None:
            return [(b * self.T, (b + 1) * self.T) for b in range(self.B)]
        c = self.cu_seqlens
        return [(int(c[i]), int(c[i + 1])) for i in range(len(c) - 1)]


def _maybe_bf16(x: np.ndarray, in_dtype: str) -> np.ndarray:
    return bf16_round(x) if in_dtype == "bf16" else x.astype(np.float32)


def make_prefill(seed: int, B: int, T: int, H: int, dk: int, dv: int,
                 in_dtype: str = "bf16", gscale: float = 1.0,
                 h0_std: Optional[float] = None,
                 seqlens: Optional[np.ndarray] = None,
                 lengths_range: Optional[tuple] = None, n_seqs: int = 0,
                 name: str = "", fused: bool = False, scalar_gate: bool = False) -> KdaInputs:
    """Draw one prefill problem.

    For packed variable-length input either pass ``seqlens`` or
    ``lengths_range=(lo, hi)`` with ``n_seqs`` (lengths uniform on the
    inclusive range, drawn first); then B must be 1 and T is their sum.
    """
    rng = np.random.default_rng(seed)
    cu = None
    if lengths_range is not None:
        lo, hi = lengths_range
        seqlens = rng.integers(lo, hi + 1, size=n_seqs)
    if seqlens is not None:
        seqlens = np.asarray(seqlens, dtype=np.int64)
        cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(seqlens)
        B, T = 1, int(cu[-1])
    N = B if cu is None else len(cu) - 1
    f32 = np.float32
    q = rng.standard_normal((B, T, H, dk), dtype=f32)
    k = rng.standard_normal((B, T, H, dk), dtype=f32)
    v = rng.standard_normal((B, T, H, dv), dtype=f32)
    bl = rng.standard_normal((B, T, H), dtype=f32)
    gl = rng.standard_normal((B, T, H) if scalar_gate else (B, T, H, dk), dtype=f32)
    h0 = None
    if h0_std is not None:
        h0 = (h0_std * rng.standard_normal((N, H, dk, dv), dtype=f32)).astype(f32)
    q = _maybe_bf16(q if fused else l2_normalise(q), in_dtype)
    k = _maybe_bf16(k if fused else l2_normalise(k), in_dtype)
    v = _maybe_bf16(v, in_dtype)
    beta = _maybe_bf16(sigmoid(bl), in_dtype)
    g = gl if fused else (-np.float32(gscale) * softplus(gl)).astype(f32)
    return KdaInputs(q=q, k=k, v=v, g=g, beta=beta, h0=h0, cu_seqlens=cu,
                     in_dtype=in_dtype, name=name,
                     meta=dict(seed=seed, gscale=gscale, h0_std=h0_std), fused=fused,
                     scalar_gate=scalar_gate)


def make_dplr(seed: int, B: int, T: int, H: int, dk: int, dv: int, in_dtype: str = "bf16",
              gscale: float = 1.0, h0_std: Optional[float] = None, seqlens=None) -> dict:
    """Inputs of the general DPLR recurrence S_t = (Diag(e^g) - a b^T) S + k v^T.

    Draw order: [lengths], q, k, v, beta-logits, g-logits, w, h0, where w is a
    second unit direction per token and head.  q, k, w are L2-normalised N(0,1),
    v ~ N(0,1), g = -gscale softplus(N(0,1)) and beta = sigmoid(N(0,1)), as in
    make_prefill; then a = beta w and b = e^g * w, so the transition
    Diag(e^g) - a b^T = (I - beta w w^T) Diag(e^g) contracts while a and b are
    untied from the key k of the write (which is beta k).  Values that travel
    in in_dtype are rounded once; b is formed from the rounded w.  Returns a dict
    of float32 arrays q, k, v, g, a, b [B, T, H, d], h0 or None, cu_seqlens or
    None, and in_dtype."""
    rng = np.random.default_rng(seed)
    cu = None
    if seqlens is not None:
        seqlens = np.asarray(seqlens, dtype=np.int64)
        cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(seqlens)
        B, T = 1, int(cu[-1])
    N = B if cu is None else len(cu) - 1
    f32 = np.float32
    q = rng.standard_normal((B, T, H, dk), dtype=f32)
    k = rng.standard_normal((B, T, H, dk), dtype=f32)
    v = rng.standard_normal((B, T, H, dv), dtype=f32)
    bl = rng.standard_normal((B, T, H), dtype=f32)
    gl = rng.standard_normal((B, T, H, dk), dtype=f32)
    w = rng.standard_normal((B, T, H, dk), dtype=f32)
    h0 = None if h0_std is None else (h0_std * rng.standard_normal((N, H, dk, dv), dtype=f32)).astype(f32)
    beta = sigmoid(bl)[..., None]
    g = (-np.float32(gscale) * softplus(gl)).astype(f32)
    wr = _maybe_bf16(l2_normalise(w), in_dtype)
    return dict(q=_maybe_bf16(l2_normalise(q), in_dtype), k=_maybe_bf16(beta * l2_normalise(k), in_dtype),
                v=_maybe_bf16(v, in_dtype), g=g, a=_maybe_bf16(beta * wr, in_dtype),
                b=_maybe_bf16((np.exp(g) * wr).astype(f32), in_dtype), h0=h0, cu_seqlens=cu, in_dtype=in_dtype)


def make_output_grads(x: KdaInputs, seed: int, dhT_std: Optional[float] = 0.02):
    """Loss gradients for a backward pass over problem ``x``: grad_o ~ N(0, 1)
    [B, T, H, dv] in x's input dtype (bf16-rounded for "bf16"), and the
    final-state gradient ~ N(0, dhT_std^2) [N, H, dk, dv] float32 (None when
    dhT_std is None).  Drawn from their own generator, grad_o first."""
    rng = np.random.default_rng(seed)
    do = _maybe_bf16(rng.standard_normal((x.B, x.T, x.H, x.dv), dtype=np.float32), x.in_dtype)
    dhT = None
    if dhT_std is not None:
        dhT = (dhT_std * rng.standard_normal((x.N, x.H, x.dk, x.dv), dtype=np.float32)).astype(np.float32)
    return do, dhT


def make_decode_state(seed: int, N: int, H: int, dk: int, dv: int,
                      std: float = 0.02):
    """Return (rng, S0) for the decode workload; S0 is [N, H, dk, dv] float32."""
    rng = np.random.default_rng(seed)
    s0 = (std * rng.standard_normal((N, H, dk, dv), dtype=np.float32)).astype(np.float32)
    return rng, s0


def decode_steps(rng, steps: int, N: int, H: int, dk: int, dv: int,
                 in_dtype: str = "bf16", gscale: float = 1.0, fused: bool = False,
                 scalar_gate: bool = False) -> Iterator[dict]:
    """Yield one token per sequence per step: q, k, g [N,H,dk]; v [N,H,dv]; beta [N,H].
    ``fused`` and ``scalar_gate`` (g [N,H]) as for make_prefill."""
    f32 = np.float32
    for _ in range(steps):
        q = rng.standard_normal((N, H, dk), dtype=f32)
        k = rng.standard_normal((N, H, dk), dtype=f32)
        v = rng.standard_normal((N, H, dv), dtype=f32)
        bl = rng.standard_normal((N, H), dtype=f32)
        gl = rng.standard_normal((N, H) if scalar_gate else (N, H, dk), dtype=f32)
        yield dict(q=_maybe_bf16(q if fused else l2_normalise(q), in_dtype),
                   k=_maybe_bf16(k if fused else l2_normalise(k), in_dtype),
                   v=_maybe_bf16(v, in_dtype),
                   beta=_maybe_bf16(sigmoid(bl), in_dtype),
                   g=gl if fused else (-f32(gscale) * softplus(gl)).astype(f32))


def decode_step_pool(rng, pool: int, N: int, H: int, dk: int, dv: int,
                     in_dtype: str = "bf16", gscale: float = 1.0, fused: bool = False,
                     scalar_gate: bool = False) -> dict:
    """Draw ``pool`` token batches for the decode workload, stacked on a
    leading axis: q, k, g [pool,N,H,dk]; v [pool,N,H,dv]; beta [pool,N,H].
    Step s of a long decode run uses batch s % pool (each step still reads
    its own copy at its own device offset)."""
    steps = list(decode_steps(rng, pool, N, H, dk, dv, in_dtype, gscale, fused, scalar_gate))
    return {k: np.stack([s[k] for s in steps]) for k in steps[0]}


# The five workloads: shapes and recipes of the Kimi Linear operator sweep
# (batch 1, 16 heads, head dim 128) plus a small fp32 case, a decode batch and
# a packed variable-length batch.
WORKLOADS = {
    "fp32_small": dict(kind="prefill", seed=0, B=1, T=256, H=2, dk=64, dv=64,
                       in_dtype="fp32", gscale=1.0, h0_std=None),
    "prefill_4k": dict(kind="prefill", seed=1, B=1, T=4096, H=16, dk=128, dv=128,
                       in_dtype="bf16", gscale=1.0, h0_std=None),
    "prefill_64k": dict(kind="prefill", seed=2, B=1, T=65536, H=16, dk=128, dv=128,
                        in_dtype="bf16", gscale=1.0, h0_std=0.02),
    # the same problem handed over before the L2 norm and the gate activation
    "prefill_64k_fused": dict(kind="prefill", seed=2, B=1, T=65536, H=16, dk=128, dv=128,
                              in_dtype="bf16", gscale=1.0, h0_std=0.02, fused=True),
    # the same shapes with one gate per token and head (Gated DeltaNet's gate)
    "prefill_64k_scalar_gate": dict(kind="prefill", seed=2, B=1, T=65536, H=16, dk=128, dv=128,
                                    in_dtype="bf16", gscale=1.0, h0_std=0.02, scalar_gate=True),
    "decode_256x16": dict(kind="decode", seed=3, N=256, H=16, dk=128, dv=128,
                          in_dtype="bf16", gscale=1.0, steps=1024, pool=32, state_std=0.02),
    "append_256x16x64": dict(kind="prefill", seed=5, B=256, T=64, H=16, dk=128, dv=128,
                             in_dtype="bf16", gscale=1.0, h0_std=0.02),
    # a training batch for the gradients: 16 sequences of 4096 tokens (grad_o and the
    # final-state gradient from make_output_grads with seed + 100)
    "backward_16x4096x16": dict(kind="prefill", seed=6, B=16, T=4096, H=16, dk=128, dv=128,
                                in_dtype="bf16", gscale=1.0, h0_std=0.02),
    # the gradients of the prefill shape: one sequence of 65,536 tokens
    "backward_64k": dict(kind="prefill", seed=2, B=1, T=65536, H=16, dk=128, dv=128,
                         in_dtype="bf16", gscale=1.0, h0_std=0.02),
    "varlen_8seq": dict(kind="prefill", seed=4, B=1, T=None, H=32, dk=128, dv=128,
                        in_dtype="bf16", gscale=0.01, h0_std=0.02,
                        lengths_range=(1024, 32768), n_seqs=8),
}


def make_workload(name: str) -> KdaInputs:
    """Draw one of the named prefill workloads."""
    w = dict(WORKLOADS[name])
    if w.pop("kind") != "prefill":
        raise ValueError(f"{name} is not a prefill workload")
    T = w.pop("T")
    return make_prefill(T=T if T is not None else 0, name=name, **w)
