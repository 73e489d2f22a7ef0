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
    ok, hk = kda.recurrent_fwd(f(x.q), f(x.k), f(x.v), f(x.g), f(x.beta), initial_state=f(x.h0))
    torch.cuda.synchronize()
    eo, es = rel(od.cpu().numpy(), ok.cpu().numpy()), rel(hd.cpu().numpy(), hk.cpu().numpy())
    say(f"case dplr_kda_case: o={eo:.2e} state={es:.2e}")
    assert eo <= TOL_FP32 and es <= TOL_FP32


def test_dplr_heads_grouped_per_xcd(kda):
    """4 sequences x 8 heads (32 = 4 x 8 sequence-heads): the kernel maps
    workgroups so that a head's dv slices share one XCD, over several groups
    of 8; parity is unchanged."""
    check(kda, make_dplr(163, 4, 20, 8, 128, 128, h0_std=0.3), "dplr_grouped", scale=0.9)
