"""GPU parity of the recurrent backward (kda_recurrent_bwd) against the fp64
oracle's gradients (oracle.backward, itself pinned by finite differences and
closed forms in test_oracle_backward.py).

Gate (kda_testlib.Gate): per (sequence, head) slice, ||gpu - oracle||_F /
||oracle||_F for each of dq, dk, dv, dg, dbeta and dh0, and the same per row
(token rows of dq, dk, dv, dg; single tokens of dbeta; key rows of dh0), each
row against max(its own norm, the slice's RMS row norm); max-abs and rms are
printed beside them.  The kernel computes in fp32 from inputs the
oracle sees exactly (bf16 values held in float32) and writes fp32 gradients,
so the bar is the fp32 tolerance, 1e-5, for both input dtypes.
"""
import numpy as np
import pytest

import oracle
from gated_delta_rule_52_amd.inputs import make_output_grads, make_prefill, make_workload
from kda_testlib import TOL_FP32, Gate, dev, gate_all, in_dtype_of, say, upload

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


@pytest.fixture(scope="module")
def kda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_delta_rule_52_amd as m
    from gated_delta_rule_52_amd import _lib
    _lib.load()
    return m


def flat(a):
    """[B, T, H, ...] -> [B*T, H, ...]"""
    return a.reshape((-1,) + a.shape[2:])


def oracle_pair(x, do, dhT, n, h, scale):
    """The oracle's gradients for sequence n, head h alone (heads and
    sequences are independent)."""
    a, b = x.seq_bounds()[n]

    def sl(arr):
        return flat(arr)[a:b, h:h + 1][None]
    h0 = None if x.h0 is None else x.h0[n:n + 1, h:h + 1].astype(np.float64)
    dh = None if dhT is None else dhT[n:n + 1, h:h + 1].astype(np.float64)
    return oracle.backward(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), sl(do), h0=h0,
                           d_final_state=dh, scale=scale, **x.transforms())


def run_gpu(kda, x, do, dhT, scale, **kw):
    import torch
    d = upload(x)
    g = kda.recurrent_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], dev(do, in_dtype_of(x)),
                          initial_state=d["h0"], grad_final_state=None if dhT is None else dev(dhT, torch.float32),
                          cu_seqlens=d["cu"], scale=scale, **x.transforms(), **kw)
    torch.cuda.synchronize()
    return g


def add_pair(gates, g, ref, x, n, h):
    """Add the slices of (sequence n, head h) to the gates; g holds the device
    results."""
    a, b = x.seq_bounds()[n]
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        gg = flat(g[name])[a:b, h].cpu().numpy()
        gates[name].add(gg, ref[name].reshape(gg.shape))
    if g["dh0"] is not None:
        gates["dh0"].add(g["dh0"][n, h].cpu().numpy(), ref["dh0"][0, 0])


def check(kda, x, do, dhT, scale=1.0, pairs=None, tol=TOL_FP32):
    say(f"case {x.name}: B={x.B} T={x.T} H={x.H} dk={x.dk} dv={x.dv} N={x.N} dtype={x.in_dtype} "
        f"h0={x.h0 is not None} dhT={dhT is not None} scale={scale}")
    g = run_gpu(kda, x, do, dhT, scale)
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


def test_bf16_several_blocks_ragged_tail(kda):
    """dk = dv = 128, bf16, 50 tokens: six blocks of 8 stored states and a
    tail of 2, initial state and final-state gradient, scale 0.9."""
    x = make_prefill(140, 2, 50, 3, 128, 128, h0_std=0.3, name="bwd_bf16")
    do, dhT = make_output_grads(x, 240, dhT_std=0.3)
    check(kda, x, do, dhT, scale=0.9)


@pytest.mark.parametrize("dk,dv,dt", [(64, 64, "fp32"), (128, 64, "bf16"), (64, 128, "bf16"),
                                      (128, 128, "fp32")])
def test_head_dims_and_dtypes(kda, dk, dv, dt):
    x = make_prefill(141, 1, 37, 2, dk, dv, in_dtype=dt, h0_std=0.3, name=f"bwd_{dk}x{dv}_{dt}")
    do, dhT = make_output_grads(x, 241, dhT_std=0.3)
    check(kda, x, do, dhT)


def test_long_single_sequence_segmented(kda):
    """One sequence of 16384 tokens, 2 heads: cut into 128 segments that run
    in parallel, chained by the forward and reverse combines."""
    x = make_prefill(146, 1, 16384, 2, 128, 128, h0_std=0.05, name="bwd_single_16k")
    do, dhT = make_output_grads(x, 246, dhT_std=0.05)
    check(kda, x, do, dhT)


@pytest.mark.parametrize("dk,dv,dt", [(64, 64, "fp32"), (64, 128, "bf16"), (128, 64, "bf16")])
def test_varlen_long_members_segmented(kda, dk, dv, dt):
    """Packed sequences of 700, 0, 64, 65, 1, 300 tokens: several of several
    segments, with every head size."""
    x = make_prefill(147, 1, 0, 2, dk, dv, in_dtype=dt, gscale=0.1, h0_std=0.3,
                     seqlens=[700, 0, 64, 65, 1, 300], name=f"bwd_varlen_seg_{dk}x{dv}")
    do, dhT = make_output_grads(x, 247, dhT_std=0.3)
    check(kda, x, do, dhT, scale=0.8)


def test_varlen_with_empty_and_short_sequences(kda):
    """Lengths 0, 1, 7, 8, 9, 33, 0, 64, 17 in one packed batch: every block
    boundary case; empty sequences pass the final-state gradient through."""
    x = make_prefill(142, 1, 0, 2, 128, 128, h0_std=0.3, seqlens=[0, 1, 7, 8, 9, 33, 0, 64, 17],
                     name="bwd_varlen")
    do, dhT = make_output_grads(x, 242, dhT_std=0.3)
    check(kda, x, do, dhT)


def test_without_initial_state_or_final_gradient(kda):
    x = make_prefill(143, 2, 21, 2, 128, 128, name="bwd_zero_states")
    do, _ = make_output_grads(x, 243, dhT_std=None)
    check(kda, x, do, None)


def test_long_sequences(kda):
    """1500 tokens: 188 stored states per sequence, gate scale 1 (short memory)
    and 0.01 (long memory, gradients reach far back)."""
    for gs in (1.0, 0.01):
        x = make_prefill(144, 1, 1500, 2, 128, 128, gscale=gs, h0_std=0.05, name=f"bwd_long_g{gs}")
        do, dhT = make_output_grads(x, 244, dhT_std=0.05)
        check(kda, x, do, dhT)


@pytest.mark.parametrize("T", [40, 300])
def test_in_place_and_deterministic(kda, T):
    """grad_initial_state may be grad_final_state (or initial_state), for
    sequences of one segment (40 tokens) and of several (300); two runs give
    the same bits; the gradient outputs need no prior contents."""
    import torch
    x = make_prefill(145, 2, T, 2, 128, 128, h0_std=0.3, name="bwd_in_place")
    do, dhT = make_output_grads(x, 245, dhT_std=0.3)
    d = upload(x)
    dod, dht = dev(do, in_dtype_of(x)), dev(dhT, torch.float32)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], dod)
    a = kda.recurrent_bwd(*args, initial_state=d["h0"], grad_final_state=dht)
    b = kda.recurrent_bwd(*args, initial_state=d["h0"], grad_final_state=dht)
    buf = dht.clone()
    c = kda.recurrent_bwd(*args, initial_state=d["h0"], grad_final_state=buf, grad_initial_state=buf)
    h0c = d["h0"].clone()
    e = kda.recurrent_bwd(*args, initial_state=h0c, grad_final_state=dht, grad_initial_state=h0c)
    # caller-supplied gradient tensors holding garbage are overwritten entirely
    pre = {n: torch.full_like(a[n], float("nan")) for n in ("dq", "dk", "dv", "dg", "dbeta")}
    f = kda.recurrent_bwd(*args, initial_state=d["h0"], grad_final_state=dht, out=pre)
    torch.cuda.synchronize()
    for name in NAMES:
        assert torch.equal(a[name], f[name]), f"{name} differs with caller-supplied outputs"
        assert torch.equal(a[name], b[name]), f"{name} not deterministic"
        assert torch.equal(a[name], c[name]), f"{name} differs in place (grad_final_state)"
        assert torch.equal(a[name], e[name]), f"{name} differs in place (initial_state)"


def test_full_size_workload_sampled(kda):
    """The 16 x 4096 x 16 training batch in the launch configuration the
    benchmark times, checked on three (sequence, head) pairs."""
    x = make_workload("backward_16x4096x16")
    do, dhT = make_output_grads(x, 106)
    check(kda, x, do, dhT, pairs=[(0, 0), (7, 5), (15, 15)])


def test_thousands_of_short_sequences(kda):
    """3,000 packed sequences of 0 to 9 tokens, 2 heads: every block length,
    empty sequences among them; checked on a spread of sequences."""
    rng = np.random.default_rng(148)
    lens = rng.integers(0, 10, size=3000)
    x = make_prefill(148, 1, 0, 2, 64, 64, in_dtype="fp32", h0_std=0.3, seqlens=lens, name="bwd_3000")
    do, dhT = make_output_grads(x, 248, dhT_std=0.3)
    pairs = [(n, h) for n in list(range(0, 3000, 97)) + [2999] for h in range(2)]
    check(kda, x, do, dhT, pairs=pairs)


@pytest.mark.parametrize("dk,dv,dt", [(128, 128, "bf16"), (64, 64, "fp32")])
def test_scalar_gate(kda, dk, dv, dt):
    """One gate per token and head (Gated DeltaNet): dg is [B, T, H], the sum
    over key channels; 300 tokens so that sequences have several segments."""
    x = make_prefill(149, 2, 300, 2, dk, dv, in_dtype=dt, h0_std=0.3, scalar_gate=True, name=f"bwd_scalar_{dt}")
    do, dhT = make_output_grads(x, 249, dhT_std=0.3)
    check(kda, x, do, dhT, scale=0.9)


@pytest.mark.parametrize("scalar_gate,dt", [(False, "bf16"), (True, "bf16"), (False, "fp32")])
def test_input_transforms(kda, scalar_gate, dt):
    """Raw q, k and gate logits (the forward's in-kernel L2 norm and softplus
    gate): dq, dk and dg are gradients of the raw inputs, carried back through
    both transforms; several segments per sequence."""
    x = make_prefill(152, 2, 300, 2, 128, 128, in_dtype=dt, h0_std=0.3, fused=True, scalar_gate=scalar_gate,
                     name=f"bwd_transforms_{'scalar' if scalar_gate else 'channel'}_{dt}")
    do, dhT = make_output_grads(x, 252, dhT_std=0.3)
    check(kda, x, do, dhT, scale=0.9)


@pytest.mark.parametrize("dk,dv,dt", [(64, 64, "fp32"), (128, 128, "bf16")])
def test_segmented_with_heads_grouped_per_xcd(kda, dk, dv, dt):
    """2 sequences of 1,024 tokens x 8 heads (16 sequence-heads, a multiple of
    8): several segments per sequence, so the reverse combine chains them with
    a head's dv slices mapped to one XCD, over two groups of 8."""
    x = make_prefill(153, 2, 1024, 8, dk, dv, in_dtype=dt, h0_std=0.1, name=f"bwd_grouped_{dk}x{dv}")
    do, dhT = make_output_grads(x, 253, dhT_std=0.1)
    check(kda, x, do, dhT, scale=0.9)


def test_more_segments_than_a_grid_dimension(kda):
    """65,000 packed sequences of 0 to 2 tokens (dk = dv = 64, fp32): about
    66,000 segment slots, more than a grid's y dimension takes; the segment
    index lives in grid.x.  Checked on a spread of sequences."""
    rng = np.random.default_rng(154)
    lens = rng.integers(0, 3, size=65000)
    x = make_prefill(154, 1, 0, 1, 64, 64, in_dtype="fp32", h0_std=0.3, seqlens=lens, name="bwd_65000")
    do, dhT = make_output_grads(x, 254, dhT_std=0.3)
    pairs = [(n, 0) for n in list(range(0, 65000, 1297)) + [64999]]
    check(kda, x, do, dhT, pairs=pairs)
