"""GPU parity of the fused input transforms against the fp64 oracle.

Inputs come before the last two steps of the synthetic recipe (``fused=True``):
q and k unnormalised, g the gate logits.  The kernels apply the per-token L2
norm of q and k and the log-gate -gate_scale * softplus(z) themselves; the
oracle applies the same transforms in fp64.  Same gate and tolerances as
the other parity tests (kda_testlib.Gate: per (sequence, head) slice and per
row, 2e-3 for bf16 inputs, 1e-5 for fp32).
"""
import numpy as np
import pytest

import oracle
from gated_delta_rule_52_amd.inputs import decode_step_pool, make_decode_state, make_prefill
from kda_testlib import TOL_BF16, TOL_FP32, Gate, check_prefill_outputs, dev, gate_all, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_delta_rule_52_amd as m
    from gated_delta_rule_52_amd import _lib
    _lib.load()
    return m


def oracle_fused(x, heads):
    return oracle.forward(x.q, x.k, x.v, x.g, x.beta, h0=None if x.h0 is None else x.h0.astype(np.float64),
                          cu_seqlens=x.cu_seqlens, heads=heads, **x.transforms())


def check(kda, x, path="chunk"):
    import torch
    tol = TOL_FP32 if x.in_dtype == "fp32" else TOL_BF16
    heads = list(range(x.H))
    say(f"case {x.name} ({path}): B={x.B} T={x.T} H={x.H} dk={x.dk} dv={x.dv} N={x.N} "
        f"dtype={x.in_dtype} transforms={x.transforms()}")
    d = upload(x)
    extra = {} if path == "chunk" else dict(token_by_token=True)
    fn = kda.chunk_fwd if path == "chunk" else kda.recurrent_fwd
    o, hT = fn(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["h0"], cu_seqlens=d["cu"],
               out_dtype=torch.float32, **x.transforms(), **extra)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_fused(x, heads)
    check_prefill_outputs(o.cpu().numpy(), hT.cpu().numpy(), o_ref, h_ref, x, heads, tol)


def test_bf16_matrix_core_path(kda):
    """dk = dv = 128, bf16: the matrix-core prep with the transforms, several
    chunks and a ragged tail, two sequences."""
    check(kda, make_prefill(110, 2, 200, 3, 128, 128, h0_std=0.3, fused=True, name="fused_bf16"))


def test_bf16_exact_chunks(kda):
    """gate_scale 3: chunks decay past e^-80, so the pair-by-pair prep path
    runs with the transforms too."""
    check(kda, make_prefill(111, 1, 160, 2, 128, 128, gscale=3.0, h0_std=0.3, fused=True, name="fused_exact"))


@pytest.mark.parametrize("dk,dv,dt", [(64, 64, "fp32"), (128, 128, "fp32"), (64, 128, "bf16")])
def test_fp32_path(kda, dk, dv, dt):
    check(kda, make_prefill(112, 1, 150, 2, dk, dv, in_dtype=dt, h0_std=0.3, fused=True,
                            name=f"fused_{dk}x{dv}_{dt}"))


def test_varlen_long_retention(kda):
    x = make_prefill(113, 1, 0, 2, 128, 128, gscale=0.01, h0_std=0.02, fused=True,
                     seqlens=[300, 0, 1, 64, 129], name="fused_varlen")
    check(kda, x)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_recurrent_fwd(kda, dt):
    check(kda, make_prefill(114, 2, 40, 2, 128, 128, in_dtype=dt, h0_std=0.3, fused=True,
                            name=f"fused_rec_{dt}"), path="recurrent")


@pytest.mark.parametrize("dk,dv,dt", [(128, 128, "bf16"), (64, 128, "fp32")])
def test_decode_steps(kda, dk, dv, dt):
    """Eight in-place decode steps with the transforms against the oracle's
    steps (state chained in fp64)."""
    import torch
    N, H, steps, gs = 6, 3, 8, 0.5
    rng, S0 = make_decode_state(115, N, H, dk, dv, std=0.3)
    P = decode_step_pool(rng, steps, N, H, dk, dv, in_dtype=dt, fused=True)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    tol = TOL_FP32 if dt == "fp32" else TOL_BF16
    S = dev(S0, torch.float32)
    ref = S0.astype(np.float64)
    g_o, g_s = Gate("o", tol), Gate("state", tol)
    for t in range(steps):
        o = kda.recurrent_step(dev(P["q"][t], tdt), dev(P["k"][t], tdt), dev(P["v"][t], tdt),
                               dev(P["g"][t], torch.float32), dev(P["beta"][t], tdt), S,
                               out_dtype=torch.float32, qk_l2norm=True, gate_logits=True, gate_scale=gs)
        o_ref, ref = oracle.decode_step(P["q"][t], P["k"][t], P["v"][t], P["g"][t], P["beta"][t], ref,
                                        qk_l2norm=True, gate_logits=True, gate_scale=gs)
        torch.cuda.synchronize()
        og, sg = o.cpu().numpy(), S.cpu().numpy()
        for n in range(N):
            for h in range(H):
                g_o.add(og[n, h][None], o_ref[n, h][None])
                g_s.add(sg[n, h], ref[n, h])
    say(f"case decode transforms dk={dk} dv={dv} {dt}, {steps} steps")
    gate_all([g_o, g_s])


# ------------------------------------------- scalar gate (Gated DeltaNet's gate)

@pytest.mark.parametrize("fused", [False, True], ids=["log_gate", "logits_l2norm"])
def test_scalar_gate_bf16(kda, fused):
    """g of shape [B,T,H] on the matrix-core prep, alone and with both transforms."""
    check(kda, make_prefill(116, 2, 150, 2, 128, 128, h0_std=0.3, fused=fused, scalar_gate=True,
                            name=f"scalar_bf16_{'fused' if fused else 'plain'}"))


def test_scalar_gate_exact_chunks(kda):
    check(kda, make_prefill(117, 1, 130, 2, 128, 128, gscale=3.0, h0_std=0.3, scalar_gate=True,
                            name="scalar_exact"))


@pytest.mark.parametrize("dk,dv,dt", [(64, 64, "fp32"), (64, 128, "bf16")])
def test_scalar_gate_fp32_path(kda, dk, dv, dt):
    check(kda, make_prefill(118, 1, 99, 2, dk, dv, in_dtype=dt, h0_std=0.3, fused=True, scalar_gate=True,
                            name=f"scalar_{dk}x{dv}_{dt}"))


def test_scalar_gate_recurrent_fwd(kda):
    check(kda, make_prefill(119, 3, 33, 2, 128, 128, h0_std=0.3, scalar_gate=True, name="scalar_rec"),
          path="recurrent")


def test_scalar_gate_decode_step(kda):
    import torch
    N, H, dk, dv = 5, 2, 128, 64
    rng, S0 = make_decode_state(120, N, H, dk, dv, std=0.3)
    P = decode_step_pool(rng, 1, N, H, dk, dv, in_dtype="bf16", scalar_gate=True)
    S = dev(S0, torch.float32)
    o = kda.recurrent_step(dev(P["q"][0], torch.bfloat16), dev(P["k"][0], torch.bfloat16),
                           dev(P["v"][0], torch.bfloat16), dev(P["g"][0], torch.float32),
                           dev(P["beta"][0], torch.bfloat16), S, out_dtype=torch.float32, scalar_gate=True)
    o_ref, s_ref = oracle.decode_step(P["q"][0], P["k"][0], P["v"][0], P["g"][0], P["beta"][0],
                                      S0.astype(np.float64), scalar_gate=True)
    torch.cuda.synchronize()
    og, sg = o.cpu().numpy(), S.cpu().numpy()
    go, gs = Gate("o", TOL_BF16), Gate("state", TOL_BF16)
    for n in range(N):
        for h in range(H):
            go.add(og[n, h][None], o_ref[n, h][None])
            gs.add(sg[n, h], s_ref[n, h])
    say("case scalar-gate decode")
    gate_all([go, gs])
