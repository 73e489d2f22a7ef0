"""GPU parity of the chunkwise gradients (kda_chunk_bwd) against the fp64
oracle's gradients (oracle.backward, pinned by finite differences and closed
forms in test_oracle_backward.py).

Gate (kda_testlib.Gate) as for the token-level gradients: per (sequence,
head) slice and per row, for dq, dk, dv, dg, dbeta and dh0.  The state
recurrences of the chunk path run on fp16 operands with fp32 accumulation,
like the bf16 prefill, so the bar is the bf16 tolerance, 2e-3 (the pages' FLA
tests allow about 0.002 to 0.02 on gradients).
"""
import numpy as np
import pytest

from gated_delta_rule_52_amd.inputs import make_output_grads, make_prefill
from kda_testlib import TOL_BF16, Gate, dev, gate_all, say, upload
from test_gpu_backward import NAMES, add_pair, flat, oracle_pair

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_delta_rule_52_amd as m
    from gated_delta_rule_52_amd import _lib
    _lib.load()
    return m


def run_chunk(kda, x, do, dhT, scale):
    import torch
    d = upload(x)
    g = kda.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], dev(do, torch.bfloat16),
                      initial_state=d["h0"], grad_final_state=None if dhT is None else dev(dhT, torch.float32),
                      cu_seqlens=d["cu"], scale=scale)
    torch.cuda.synchronize()
    return g


def check(kda, x, do, dhT, scale=1.0, pairs=None, tol=TOL_BF16):
    say(f"case {x.name}: B={x.B} T={x.T} H={x.H} N={x.N} h0={x.h0 is not None} dhT={dhT is not None} "
        f"scale={scale}")
    g = run_chunk(kda, x, do, dhT, scale)
    pairs = pairs or [(n, h) for n in range(x.N) for h in range(x.H)]
    gates = {k: Gate(k, tol) for k in NAMES}
    for n, h in pairs:
        a, b = x.seq_bounds()[n]
        if b == a:  # an empty sequence: the initial-state gradient is the final-state gradient
            want = np.zeros((x.dk, x.dv), np.float32) if dhT is None else dhT[n, h]
            assert np.array_equal(g["dh0"][n, h].cpu().numpy(), want)
            continue
        add_pair(gates, g, oracle_pair(x, do, dhT, n, h, scale), x, n, h)
    gate_all([gates[k] for k in NAMES if gates[k].slices])
    return g


def test_chunks_and_ragged_tail(kda):
    """Two sequences of 150 tokens (two chunks and a tail of 22), 2 heads,
    initial state, final-state gradient, scale 0.9."""
    x = make_prefill(160, 2, 150, 2, 128, 128, h0_std=0.3, name="cbwd_150")
    do, dhT = make_output_grads(x, 260, dhT_std=0.3)
    check(kda, x, do, dhT, scale=0.9)


def test_long_sequence_several_segments(kda):
    """One sequence of 3000 tokens, 2 heads: many segments, chained by both
    combines."""
    x = make_prefill(161, 1, 3000, 2, 128, 128, h0_std=0.05, name="cbwd_3000")
    do, dhT = make_output_grads(x, 261, dhT_std=0.05)
    check(kda, x, do, dhT)


def test_varlen_with_empty_and_short_members(kda):
    """Packed sequences of 700, 0, 64, 65, 1, 300 tokens with long memory
    (gate scale 0.1), no final-state gradient."""
    x = make_prefill(162, 1, 0, 2, 128, 128, gscale=0.1, h0_std=0.3, seqlens=[700, 0, 64, 65, 1, 300],
                     name="cbwd_varlen")
    do, _ = make_output_grads(x, 262, dhT_std=None)
    check(kda, x, do, None)


def test_slow_decay_long_retention(kda):
    """Gate scale 0.01 over 2000 tokens: the segment transitions and the
    reverse combine carry most of the gradient."""
    x = make_prefill(163, 1, 2000, 2, 128, 128, gscale=0.01, h0_std=0.05, name="cbwd_slow")
    do, dhT = make_output_grads(x, 263, dhT_std=0.05)
    check(kda, x, do, dhT)


def test_zero_and_carrying_transitions_in_one_chain(kda):
    """4,096 tokens, 2 heads, one chunk per segment: long retention (gate scale 0.01) with every third
    chunk decaying past e^-200 (scale 4), whose transition is exactly zero.  Both combines read the
    zero transitions as zeros without fetching them and carry the others."""
    x = make_prefill(167, 1, 4096, 2, 128, 128, gscale=0.01, h0_std=0.05, name="cbwd_mixed")
    for c0 in range(0, 4096, 3 * 64):
        x.g[0, c0:c0 + 64] *= 400.0
    do, dhT = make_output_grads(x, 267, dhT_std=0.05)
    check(kda, x, do, dhT)


def test_head_and_tail_walks_that_hold_and_that_fail(kda):
    """32,768 tokens, 2 heads: segments of 8 chunks, long retention (gate scale 0.01), with strong gates (scale 3)
    in the last 4 chunks of every third segment (the forward tail walk holds) and in the first 4 chunks of the
    next one (the reverse local pass walks only those: the forward transition over them is zero); the third
    segment of each group keeps its memory end to end (both walks whole).  Two sampled pairs."""
    x = make_prefill(168, 1, 32768, 2, 128, 128, gscale=0.01, h0_std=0.05, name="cbwd_walks")
    for s0 in range(0, 32768, 3 * 512):
        x.g[0, s0 + 256:s0 + 512] *= 300.0
        x.g[0, s0 + 512:s0 + 768] *= 300.0
    do, dhT = make_output_grads(x, 268, dhT_std=0.05)
    check(kda, x, do, dhT, pairs=[(0, 0), (0, 1)])


def test_fast_decay_takes_the_exact_chunk_path(kda):
    """Gate scale 4: chunks decay past e^-80, so the Gram products and their
    gradients are formed pair by pair."""
    x = make_prefill(164, 1, 200, 2, 128, 128, gscale=4.0, h0_std=0.3, name="cbwd_fast")
    do, dhT = make_output_grads(x, 264, dhT_std=0.3)
    check(kda, x, do, dhT)


def test_no_states_and_a_scale(kda):
    """Three sequences of 333 tokens, no initial state, no final-state
    gradient, scale 0.5."""
    x = make_prefill(166, 3, 333, 2, 128, 128, name="cbwd_nostate")
    do, _ = make_output_grads(x, 266, dhT_std=None)
    check(kda, x, do, None, scale=0.5)


def test_full_size_sampled_heads(kda):
    """The timed gradients workload (one sequence of 65,536 tokens, 16 heads,
    initial state and final-state gradient) in the launch configuration the
    benchmark times, heads 0 and 11 against the oracle."""
    from gated_delta_rule_52_amd.inputs import make_workload
    x = make_workload("backward_64k")
    do, dhT = make_output_grads(x, 106)
    check(kda, x, do, dhT, pairs=[(0, 0), (0, 11)])


def test_agrees_with_the_token_path(kda):
    """The chunk path and kda_recurrent_bwd give the same gradients (within
    the bf16 tolerance) on one problem with every input."""
    import torch
    x = make_prefill(165, 1, 1000, 2, 128, 128, h0_std=0.1, name="cbwd_vs_token")
    do, dhT = make_output_grads(x, 265, dhT_std=0.1)
    gc = run_chunk(kda, x, do, dhT, 1.0)
    d = upload(x)
    gt = kda.recurrent_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], dev(do, torch.bfloat16), initial_state=d["h0"],
                           grad_final_state=dev(dhT, torch.float32))
    torch.cuda.synchronize()
    gates = {k: Gate(k, TOL_BF16) for k in NAMES}
    for h in range(x.H):
        for name in NAMES[:-1]:
            gates[name].add(flat(gc[name])[:, h].cpu().numpy(), flat(gt[name])[:, h].cpu().numpy())
        gates["dh0"].add(gc["dh0"][0, h].cpu().numpy(), gt["dh0"][0, h].cpu().numpy())
    gate_all([gates[k] for k in NAMES])
