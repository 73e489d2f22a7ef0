"""GPU parity of the general DPLR recurrence (kda_dplr_recurrent_fwd) against
the fp64 oracle (oracle.dplr_forward, pinned in test_oracle_dplr.py), with the
gate of the other parity tests (kda_testlib.Gate: per (sequence, head) slice
and per row).  The kernel computes in
fp32 from inputs the oracle sees exactly, so the bar is 1e-5 for both input
dtypes."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_52_amd.inputs import make_dplr, make_prefill
from kda_testlib import TOL_FP32, Gate, dev, gate_all, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_delta_rule_52_amd as m
    from gated_delta_rule_52_amd import _lib
    _lib.load()
    return m


def rel(x, r):
    x = np.asarray(x, np.float64)
    return float("inf") if not np.isfinite(x).all() else float(np.linalg.norm(x - r) / max(np.linalg.norm(r), 1e-30))


def check(kda, d, name, scale=1.0):
    import torch
    dt = torch.bfloat16 if d["in_dtype"] == "bf16" else torch.float32
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    say(f"case {name}: B={B} T={T} H={H} dk={dk} dv={dv} dtype={d['in_dtype']}")
    t = {n: dev(d[n], dt) for n in ("q", "k", "v", "a", "b")}
    h0 = None if d["h0"] is None else dev(d["h0"], torch.float32)
    cu = None if d["cu_seqlens"] is None else dev(d["cu_seqlens"], torch.int32)
    o, hT = kda.dplr_recurrent_fwd(t["q"], t["k"], t["v"], dev(d["g"], torch.float32), t["a"], t["b"],
                                   initial_state=h0, cu_seqlens=cu, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.dplr_forward(d["q"], d["k"], d["v"], d["g"], d["a"], d["b"], h0=d["h0"],
                                       cu_seqlens=d["cu_seqlens"], scale=scale)
    og, hg = o.cpu().numpy(), hT.cpu().numpy()
    cuv = d["cu_seqlens"] if d["cu_seqlens"] is not None else np.arange(B + 1) * T
    go, gs = Gate("o", TOL_FP32), Gate("state", TOL_FP32)
    for n in range(len(cuv) - 1):
        a0, a1 = int(cuv[n]), int(cuv[n + 1])
        for h in range(H):
            if a1 > a0:
                go.add(og.reshape(-1, H, dv)[a0:a1, h], o_ref.reshape(-1, H, dv)[a0:a1, h])
            gs.add(hg[n, h], h_ref[n, h])
    gate_all([go, gs])


@pytest.mark.parametrize("dk,dv,dt", [(128, 128, "bf16"), (64, 64, "fp32"), (128, 64, "bf16"), (64, 128, "fp32")])
def test_dplr_parity(kda, dk, dv, dt):
    check(kda, make_dplr(160, 2, 61, 3, dk, dv, in_dtype=dt, h0_std=0.3), f"dplr_{dk}x{dv}_{dt}", scale=0.8)


def test_dplr_varlen_and_no_initial_state(kda):
    check(kda, make_dplr(161, 1, 0, 2, 128, 128, seqlens=[0, 1, 17, 64, 5, 130]), "dplr_varlen")


def test_dplr_long_sequences(kda):
    check(kda, make_dplr(162, 2, 1000, 2, 128, 128, gscale=0.05, h0_std=0.05), "dplr_long")


def test_dplr_kda_case_matches_kda_kernel(kda):
    """a = beta k, b = alpha * k and write key beta k (fp32): the DPLR kernel
    gives the KDA kernel's results."""
    import torch
    x = make_prefill(163, 2, 50, 2, 128, 128, in_dtype="fp32", h0_std=0.3)
    beta = x.beta[..., None]
    a = (beta * x.k).astype(np.float32)
    b = (np.exp(x.g) * x.k).astype(np.float32)
    f = lambda z: dev(z, torch.float32)
    od, hd = kda.dplr_recurrent_fwd(f(x.q), f(a), f(x.v), f(x.g), f(a), f(b), initial_state=f(x.h0))
    ok, hk = kda.recurrent_fwd(f(x.q), f(x.k), f(x.v), f(x.g), f(x.beta), initial_state=f(x.h0), token_by_token=True)
    torch.cuda.synchronize()
    eo, es = rel(od.cpu().numpy(), ok.cpu().numpy()), rel(hd.cpu().numpy(), hk.cpu().numpy())
    say(f"case dplr_kda_case: o={eo:.2e} state={es:.2e}")
    assert eo <= TOL_FP32 and es <= TOL_FP32


def test_dplr_heads_grouped_per_xcd(kda):
    """4 sequences x 8 heads (32 = 4 x 8 sequence-heads): the kernel maps
    workgroups so that a head's dv slices share one XCD, over several groups
    of 8; parity is unchanged."""
    check(kda, make_dplr(163, 4, 20, 8, 128, 128, h0_std=0.3), "dplr_grouped", scale=0.9)


# ------------------------------------------------------------- chunkwise form

def check_chunk(kda, d, name, scale=1.0, tol=TOL_FP32):
    """kda_dplr_chunk_fwd against the fp64 oracle, with the row gate.  The
    chunk kernel computes in fp32 on matrix cores from inputs the oracle sees
    exactly, so both input dtypes are held to the fp32 tolerance."""
    import torch
    dt = torch.bfloat16 if d["in_dtype"] == "bf16" else torch.float32
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    say(f"case {name} (chunk): B={B} T={T} H={H} dk={dk} dv={dv} dtype={d['in_dtype']}")
    t = {n: dev(d[n], dt) for n in ("q", "k", "v", "a", "b")}
    h0 = None if d["h0"] is None else dev(d["h0"], torch.float32)
    cu = None if d["cu_seqlens"] is None else dev(d["cu_seqlens"], torch.int32)
    o, hT = kda.dplr_chunk_fwd(t["q"], t["k"], t["v"], dev(d["g"], torch.float32), t["a"], t["b"],
                               initial_state=h0, cu_seqlens=cu, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.dplr_forward(d["q"], d["k"], d["v"], d["g"], d["a"], d["b"], h0=d["h0"],
                                       cu_seqlens=d["cu_seqlens"], scale=scale)
    og, hg = o.cpu().numpy(), hT.cpu().numpy()
    cuv = d["cu_seqlens"] if d["cu_seqlens"] is not None else np.arange(B + 1) * T
    go, gs = Gate("o", tol), Gate("state", tol)
    for n in range(len(cuv) - 1):
        a0, a1 = int(cuv[n]), int(cuv[n + 1])
        for h in range(H):
            if a1 > a0:
                go.add(og.reshape(-1, H, dv)[a0:a1, h], o_ref.reshape(-1, H, dv)[a0:a1, h])
            gs.add(hg[n, h], h_ref[n, h])
    gate_all([go, gs])
    return o, hT


@pytest.mark.parametrize("dk,dv,dt", [(128, 128, "bf16"), (64, 64, "fp32"), (128, 64, "bf16"), (64, 128, "fp32"),
                                      (128, 128, "fp32")])
def test_dplr_chunk_parity(kda, dk, dv, dt):
    """Several chunks of 32 and a ragged tail, initial state, scale 0.8."""
    check_chunk(kda, make_dplr(170, 2, 109, 3, dk, dv, in_dtype=dt, h0_std=0.3), f"dplr_chunk_{dk}x{dv}_{dt}",
                scale=0.8)


def test_dplr_chunk_varlen_and_no_initial_state(kda):
    """Packed sequences of 0 to 130 tokens without an initial state: empty
    sequences' final state is zero, partial chunks at every length class."""
    check_chunk(kda, make_dplr(171, 1, 0, 2, 128, 128, seqlens=[0, 1, 17, 32, 33, 64, 5, 130, 0]),
                "dplr_chunk_varlen")


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
def test_dplr_chunk_long_retention_several_segments(kda, dt):
    """Slow decay (gate scale 0.05) over 1,500 and 2,000 tokens, and a packed
    batch around them: sequences cut into several segments whose transitions P
    stay far from zero, so the combine's use of P decides every later output."""
    check_chunk(kda, make_dplr(172, 2, 1500, 2, 128, 128, in_dtype=dt, gscale=0.05, h0_std=0.05),
                f"dplr_chunk_long_{dt}")
    check_chunk(kda, make_dplr(173, 1, 0, 2, 64, 64, in_dtype=dt, gscale=0.05, h0_std=0.05,
                               seqlens=[2000, 3, 0, 700]), f"dplr_chunk_long_varlen_{dt}")


def test_dplr_chunk_extreme_gates(kda):
    """Blocks of 16 rows that decay by far more than exp(80) in some channels
    take the pair-by-pair Gram entries; a chunk without decay beside them."""
    d = make_dplr(174, 1, 160, 2, 128, 128, in_dtype="fp32", h0_std=0.3)
    d["g"][0, 3:20, :, :40] = -9.0     # 17 rows x -9 in 40 channels: ranges of ~150 per 16-row block
    d["g"][0, 64:96] = 0.0             # a chunk of 32 without decay
    check_chunk(kda, d, "dplr_chunk_extreme")


def test_dplr_chunk_equals_token_kernel_and_in_place(kda):
    """The chunk form gives the token-level kernel's results (both fp32); the
    final state may alias the initial state."""
    import torch
    d = make_dplr(175, 3, 77, 2, 128, 128, in_dtype="fp32", h0_std=0.3)
    f = lambda z: dev(z, torch.float32)
    args = (f(d["q"]), f(d["k"]), f(d["v"]), f(d["g"]), f(d["a"]), f(d["b"]))
    ot, ht = kda.dplr_recurrent_fwd(*args, initial_state=f(d["h0"]))
    S = f(d["h0"])
    oc, _ = kda.dplr_chunk_fwd(*args, initial_state=S, final_state=S)
    torch.cuda.synchronize()
    eo, es = rel(oc.cpu().numpy(), ot.cpu().numpy()), rel(S.cpu().numpy(), ht.cpu().numpy())
    say(f"case dplr chunk vs token: o={eo:.2e} state={es:.2e}")
    assert eo <= TOL_FP32 and es <= TOL_FP32


def test_dplr_chunk_kda_case_matches_kda_chunk(kda):
    """a = beta k, b = alpha * k and write key beta k: the DPLR chunk kernel
    gives the KDA chunk kernel's results (fp32 path, chunk 32)."""
    import torch
    x = make_prefill(176, 2, 150, 2, 128, 128, in_dtype="fp32", h0_std=0.3)
    beta = x.beta[..., None]
    a = (beta * x.k).astype(np.float32)
    b = (np.exp(x.g) * x.k).astype(np.float32)
    f = lambda z: dev(z, torch.float32)
    od, hd = kda.dplr_chunk_fwd(f(x.q), f(a), f(x.v), f(x.g), f(a), f(b), initial_state=f(x.h0))
    ok, hk = kda.chunk_fwd(f(x.q), f(x.k), f(x.v), f(x.g), f(x.beta), initial_state=f(x.h0), chunk_size=32,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    eo, es = rel(od.cpu().numpy(), ok.cpu().numpy()), rel(hd.cpu().numpy(), hk.cpu().numpy())
    say(f"case dplr chunk, KDA case: o={eo:.2e} state={es:.2e}")
    assert eo <= TOL_FP32 and es <= TOL_FP32
