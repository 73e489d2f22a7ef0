"""GPU parity of the multi-token fused recurrent forward (kda_recurrent_fwd)
against the fp64 oracle, with the metric and tolerances of the prefill
parity tests (kda_testlib.Gate): per (sequence, head) slice and per row, for o
and the final state, at most 2e-3 for bf16 inputs and 1e-5 for fp32.
"""
import numpy as np
import pytest

from gated_delta_rule_52_amd.inputs import bf16_round, make_prefill
from kda_testlib import TOL_BF16, TOL_FP32, check_prefill_outputs, oracle_forward, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_delta_rule_52_amd as m
    from gated_delta_rule_52_amd import _lib
    _lib.load()
    return m


def run(kda, x, scale=1.0, out_dtype=None, initial=True, token_by_token=True):
    import torch
    d = upload(x)
    o, hT = kda.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                              initial_state=d["h0"] if initial else None, cu_seqlens=d["cu"],
                              scale=scale, out_dtype=out_dtype or torch.float32, token_by_token=token_by_token)
    torch.cuda.synchronize()
    return o, hT


def check(kda, x, scale=1.0, token_by_token=True):
    tol = TOL_FP32 if x.in_dtype == "fp32" else TOL_BF16
    heads = list(range(x.H))
    say(f"case {x.name}: B={x.B} T={x.T} H={x.H} dk={x.dk} dv={x.dv} N={x.N} dtype={x.in_dtype} "
        f"token_by_token={token_by_token}")
    o, hT = run(kda, x, scale=scale, token_by_token=token_by_token)
    o_ref, h_ref = oracle_forward(x, heads, scale=scale)
    check_prefill_outputs(o.cpu().numpy(), hT.cpu().numpy(), o_ref, h_ref, x, heads, tol)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64)])
def test_short_appends_bf16(kda, dk, dv):
    check(kda, make_prefill(81, 2, 64, 4, dk, dv, h0_std=0.3, name="append64"), scale=0.9)


def test_fp32_inputs(kda):
    check(kda, make_prefill(82, 1, 37, 2, 64, 64, in_dtype="fp32", h0_std=0.3, name="fp32_37"))


def test_single_token_and_no_initial_state(kda):
    check(kda, make_prefill(83, 3, 1, 2, 128, 128, name="one_token"))


def test_varlen_with_empty_and_short_sequences(kda):
    x = make_prefill(84, 1, 0, 3, 128, 128, h0_std=0.3, seqlens=[0, 1, 17, 64, 5, 40, 0], name="varlen_short")
    check(kda, x)
    o, hT = run(kda, x)
    # empty sequences carry their initial state through unchanged
    for n in (0, 6):
        assert np.array_equal(hT[n].cpu().numpy(), x.h0[n])


def test_in_place_state_and_bf16_output(kda):
    """final_state may alias initial_state; bf16 output is the fp32 output
    rounded to nearest even; two runs give the same bits."""
    import torch
    x = make_prefill(85, 2, 48, 2, 128, 128, h0_std=0.3, name="in_place")
    d = upload(x)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    o32a, ha = kda.recurrent_fwd(*args, initial_state=d["h0"], out_dtype=torch.float32, token_by_token=True)
    o32b, hb = kda.recurrent_fwd(*args, initial_state=d["h0"], out_dtype=torch.float32, token_by_token=True)
    S = d["h0"].clone()
    o16, _ = kda.recurrent_fwd(*args, initial_state=S, final_state=S, out_dtype=torch.bfloat16, token_by_token=True)
    torch.cuda.synchronize()
    assert torch.equal(o32a, o32b) and torch.equal(ha, hb), "not deterministic"
    assert torch.equal(S, ha), "in-place final state differs"
    assert np.array_equal(bf16_round(o32a.cpu().numpy()), o16.float().cpu().numpy())


@pytest.mark.parametrize("dk,dv,dt", [(128, 128, "bf16"), (64, 128, "fp32"), (128, 64, "bf16"), (64, 64, "fp32")])
def test_one_token_per_sequence_runs_as_a_decode_step(kda, dk, dv, dt):
    """Fixed-length input of one token per sequence takes the decode kernel:
    parity against the oracle from an initial state, the in-place form (final
    state aliasing the initial state) bit-equal to separate buffers, and the
    same bits as kda_recurrent_step on the same token."""
    import torch
    x = make_prefill(86, 5, 1, 3, dk, dv, in_dtype=dt, h0_std=0.3, name=f"one_token_{dk}x{dv}_{dt}")
    check(kda, x, scale=0.8)
    d = upload(x)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    o1, h1 = kda.recurrent_fwd(*args, initial_state=d["h0"], scale=0.8, out_dtype=torch.float32)
    S = d["h0"].clone()
    o2, _ = kda.recurrent_fwd(*args, initial_state=S, final_state=S, scale=0.8, out_dtype=torch.float32)
    step_in = [a[:, 0].contiguous() for a in args]  # [N, H, ...]: one token per sequence
    o3 = kda.recurrent_step(*step_in, d["h0"].clone(), scale=0.8, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, S), "in-place run differs"
    assert torch.equal(o1[:, 0], o3), "differs from the decode step"


@pytest.mark.parametrize("scalar_gate", [False, True], ids=["channel_gate", "scalar_gate"])
def test_one_token_per_sequence_with_transforms(kda, scalar_gate):
    """Raw q, k and gate logits, one token per sequence: the in-kernel L2 norm
    and softplus gate give the same bits as the decode step on the same raw
    token, and the state update matches the oracle's."""
    import torch
    import oracle
    x = make_prefill(87, 4, 1, 2, 128, 128, h0_std=0.3, fused=True, scalar_gate=scalar_gate,
                     name=f"one_token_fused_{'scalar' if scalar_gate else 'channel'}")
    d = upload(x)
    tr = x.transforms()
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    o1, h1 = kda.recurrent_fwd(*args, initial_state=d["h0"], out_dtype=torch.float32, **tr)
    state = d["h0"].clone()
    o3 = kda.recurrent_step(*[a[:, 0].contiguous() for a in args], state, out_dtype=torch.float32, **tr)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, 0], o3) and torch.equal(h1, state), "differs from the decode step"
    heads = list(range(x.H))
    o_ref, h_ref = oracle.forward(x.q, x.k, x.v, x.g, x.beta, h0=x.h0.astype(np.float64), heads=heads, **tr)
    say("  one token with transforms")
    check_prefill_outputs(o1.cpu().numpy(), h1.cpu().numpy(), o_ref, h_ref, x, heads, TOL_BF16)


@pytest.mark.parametrize("dk,dv,dt", [(128, 128, "bf16"), (64, 64, "fp32")])
def test_heads_grouped_per_xcd(kda, dk, dv, dt):
    """4 sequences x 8 heads (32 sequence-heads, a multiple of 8): workgroups
    are mapped so that a head's dv slices share one XCD, over several groups
    of 8; parity is unchanged."""
    check(kda, make_prefill(88, 4, 20, 8, dk, dv, in_dtype=dt, h0_std=0.3, name=f"grouped_{dk}x{dv}"), scale=0.9)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_long_appends_take_the_chunk_path(kda, dt):
    """More than 16 tokens per sequence with a chunk workspace: kda_recurrent_fwd
    runs kda_chunk_fwd, with the same bits as calling it directly, and the
    result passes the oracle's gate; without a workspace the token kernel runs
    (and passes too)."""
    import torch
    x = make_prefill(89, 4, 48, 2, 128, 128, in_dtype=dt, h0_std=0.3, name=f"routed_{dt}")
    check(kda, x, scale=0.9, token_by_token=False)
    check(kda, x, scale=0.9, token_by_token=True)
    d = upload(x)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    o_r, h_r = kda.recurrent_fwd(*args, initial_state=d["h0"], scale=0.9, out_dtype=torch.float32)
    o_c, h_c = kda.chunk_fwd(*args, initial_state=d["h0"], scale=0.9, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o_r, o_c) and torch.equal(h_r, h_c), "routed call differs from kda_chunk_fwd"
