"""Pins for the fp64 oracle (CPU only).

The oracle is checked against facts that the pages and the mathematics fix,
never against itself:

* a two-token example worked by hand (tests/golden);
* a brute force with explicit dk x dk transition matrices;
* the reduction chain on the Kimi Linear pages: alpha = 1 and beta = 0 freezes
  the state, orthonormal keys with alpha = beta = 1 give vanilla linear
  attention, alpha = 1 gives DeltaNet, channel-uniform alpha gives Gated
  DeltaNet, and beta = 1 with a unit key read right after its write returns v;
* the beta = 0 closed form, chunk-size invariance of the chunkwise form,
  splitting a sequence at a state boundary, linearity in (V, S_0), dv-column
  independence, packed variable length, and the norm bound of the update.

Each pin is a function of a forward callable so that the same pins can be run
on deliberately broken copies of the recurrence (planted on the CPU) to show
that every plausible mistake is caught by at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import reference as ref
from gated_delta_rule_52_amd.inputs import make_prefill, bf16_round

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def hadamard_keys(dk, T, seed):
    """Rows of a Sylvester Hadamard matrix scaled to unit norm: exactly
    orthonormal in binary floating point (entries are +-1/sqrt(dk), dk = 4^m)."""
    Hm = np.array([[1.0]])
    while Hm.shape[0] < dk:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    rng = np.random.default_rng(seed)
    rows = rng.permutation(dk)[:T]
    return (Hm[rows] / np.sqrt(dk)).astype(np.float32)


def small(seed, T=13, H=2, dk=5, dv=3, h0=True, gscale=1.0):
    x = make_prefill(seed, 1, T, H, dk, dv, in_dtype="fp32", gscale=gscale,
                     h0_std=0.5 if h0 else None)
    return x


def run(fwd, x, **kw):
    return fwd(x.q, x.k, x.v, x.g, x.beta, h0=x.h0, cu_seqlens=x.cu_seqlens, **kw)


# --------------------------------------------------------------------------- pins

def pin_golden(fwd):
    d = json.load(open(os.path.join(GOLDEN, "handworked_two_tokens.json")))
    k = np.array(d["k"], np.float32)[None, :, None, :]
    v = np.array(d["v"], np.float32)[None, :, None, :]
    q = np.array(d["q"], np.float32)[None, :, None, :]
    beta = np.array(d["beta"], np.float32)[None, :, None]
    g = np.log(np.array(d["alpha"], np.float64)).astype(np.float32)[None, :, None, :]
    S0 = np.array(d["S0"], np.float64)[None, None]
    o, hT = fwd(q, k, v, g, beta, h0=S0)
    return max(rel(o[0, :, 0], d["expected_o"]), rel(hT[0, 0], d["expected_S"])) < 1e-6


def pin_dense(fwd):
    x = small(11, T=13, H=2, dk=5, dv=3)
    o, hT = run(fwd, x, scale=0.7)
    o2, S2 = ref.kda_dense_transition(x.q[0], x.k[0], x.v[0], x.g[0], x.beta[0], x.h0[0], scale=0.7)
    return max(rel(o[0], o2), rel(hT[0], S2)) < 1e-12


def pin_frozen(fwd):
    x = small(12, T=9, H=2, dk=4, dv=6)
    x.g[:] = 0.0
    x.beta[:] = 0.0
    o, hT = run(fwd, x, scale=1.3)
    want_o = 1.3 * np.einsum("hij,thi->thj", x.h0[0].astype(np.float64), x.q[0].astype(np.float64))
    return rel(o[0], want_o) < 1e-14 and rel(hT[0], x.h0[0]) < 1e-15


def pin_linear_attention(fwd):
    dk, T = 16, 16
    x = small(13, T=T, H=1, dk=dk, dv=5, h0=False)
    x.k[0, :, 0] = hadamard_keys(dk, T, 13)
    x.g[:] = 0.0
    x.beta[:] = 1.0
    o, _ = run(fwd, x)
    return rel(o[0], ref.linear_attention(x.q[0], x.k[0], x.v[0])) < 1e-13


def pin_deltanet(fwd):
    x = small(14, T=17, H=2, dk=6, dv=4)
    x.g[:] = 0.0
    o, hT = run(fwd, x)
    o2, S2 = ref.deltanet(x.q[0], x.k[0], x.v[0], x.beta[0], x.h0[0])
    return max(rel(o[0], o2), rel(hT[0], S2)) < 1e-12


def pin_gdn(fwd):
    x = small(15, T=17, H=2, dk=6, dv=4)
    x.g[:] = x.g[..., :1]                    # one forget rate per token and head
    o, hT = run(fwd, x)
    alpha = np.exp(x.g[0, :, :, 0].astype(np.float64))
    o2, S2 = ref.gated_deltanet(x.q[0], x.k[0], x.v[0], alpha, x.beta[0], x.h0[0])
    return max(rel(o[0], o2), rel(hT[0], S2)) < 1e-12


def pin_write_read(fwd):
    dk, T = 16, 40
    x = small(16, T=T, H=2, dk=dk, dv=7)
    rng = np.random.default_rng(16)
    for h in range(2):
        rows = rng.integers(0, dk, size=T)
        Hk = hadamard_keys(dk, dk, 100 + h)[rows]
        Hk *= rng.choice([-1.0, 1.0], size=(T, 1)).astype(np.float32)
        x.k[0, :, h] = Hk
    x.q[:] = x.k
    x.beta[:] = 1.0
    o, _ = run(fwd, x)
    return rel(o[0], x.v[0]) < 1e-12


def pin_decay_only(fwd):
    x = small(17, T=21, H=2, dk=5, dv=4)
    x.beta[:] = 0.0
    o, hT = run(fwd, x, scale=0.9)
    o2, S2 = ref.decay_only(x.q[0], x.g[0], x.h0[0], scale=0.9)
    return max(rel(o[0], o2), rel(hT[0], S2)) < 1e-12


def pin_chunk_invariance(fwd):
    x = small(18, T=150, H=2, dk=12, dv=7)
    o, hT = run(fwd, x, scale=0.8)
    worst = 0.0
    for C in (1, 2, 3, 7, 16, 32, 64):
        o2, S2 = ref.kda_chunked(x.q[0], x.k[0], x.v[0], x.g[0], x.beta[0], x.h0[0], scale=0.8, C=C)
        worst = max(worst, rel(o[0], o2), rel(hT[0], S2))
    return worst < 1e-11


def pin_state_split(fwd):
    x = small(19, T=50, H=2, dk=6, dv=5)
    o, hT = run(fwd, x)
    T1 = 23
    o1, h1 = fwd(x.q[:, :T1], x.k[:, :T1], x.v[:, :T1], x.g[:, :T1], x.beta[:, :T1], h0=x.h0)
    o2, h2 = fwd(x.q[:, T1:], x.k[:, T1:], x.v[:, T1:], x.g[:, T1:], x.beta[:, T1:], h0=h1)
    return max(rel(np.concatenate([o1, o2], axis=1), o), rel(h2, hT)) < 1e-12


def pin_linearity(fwd):
    x = small(20, T=30, H=2, dk=6, dv=5)
    rng = np.random.default_rng(20)
    V1 = (rng.integers(-64, 65, size=x.v.shape) / 64.0).astype(np.float32)
    V2 = (rng.integers(-64, 65, size=x.v.shape) / 64.0).astype(np.float32)
    S1 = rng.standard_normal(x.h0.shape)
    S2 = rng.standard_normal(x.h0.shape)
    oa, ha = fwd(x.q, x.k, V1, x.g, x.beta, h0=S1)
    ob, hb = fwd(x.q, x.k, V2, x.g, x.beta, h0=S2)
    oc, hc = fwd(x.q, x.k, 2 * V1 - V2, x.g, x.beta, h0=2 * S1 - S2)
    return max(rel(oc, 2 * oa - ob), rel(hc, 2 * ha - hb)) < 1e-12


def pin_column_perm(fwd):
    x = small(21, T=25, H=2, dk=6, dv=5)
    perm = np.array([3, 0, 4, 1, 2])
    o, hT = run(fwd, x)
    o2, h2 = fwd(x.q, x.k, x.v[..., perm], x.g, x.beta, h0=x.h0[..., perm])
    return max(rel(o2, o[..., perm]), rel(h2, hT[..., perm])) < 1e-14


def pin_varlen(fwd):
    lens = [7, 1, 19, 0, 12]
    x = make_prefill(22, 1, 0, 2, 5, 4, in_dtype="fp32", h0_std=0.5, seqlens=lens)
    o, hT = run(fwd, x)
    worst = 0.0
    for n, (a, b) in enumerate(x.seq_bounds()):
        on, hn = fwd(x.q[:, a:b], x.k[:, a:b], x.v[:, a:b], x.g[:, a:b], x.beta[:, a:b], h0=x.h0[n:n + 1])
        if b > a:
            worst = max(worst, rel(o[:, a:b], on))
        worst = max(worst, rel(hT[n], hn[0]))
    return worst < 1e-13


def pin_bounded(fwd):
    """||(I - b k k^T) Diag(a)|| <= 1 for unit k, b in [0,1], a <= 1, so the
    state norm grows by at most beta |k| |v| per token."""
    x = small(23, T=30, H=2, dk=6, dv=5)
    S = x.h0.astype(np.float64)
    for t in range(x.T):
        sl = slice(t, t + 1)
        _, Sn = fwd(x.q[:, sl], x.k[:, sl], x.v[:, sl], x.g[:, sl], x.beta[:, sl], h0=S)
        for h in range(x.H):
            bound = np.linalg.norm(S[0, h]) + x.beta[0, t, h] * np.linalg.norm(x.k[0, t, h].astype(np.float64)) \
                * np.linalg.norm(x.v[0, t, h].astype(np.float64))
            if np.linalg.norm(Sn[0, h]) > bound * (1 + 1e-12):
                return False
        S = Sn
    return True


PINS = [pin_golden, pin_dense, pin_frozen, pin_linear_attention, pin_deltanet, pin_gdn,
        pin_write_read, pin_decay_only, pin_chunk_invariance, pin_state_split,
        pin_linearity, pin_column_perm, pin_varlen, pin_bounded]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    assert pin(oracle.forward)


# ------------------------------------------------- planted mistakes (CPU, numpy)

def make_recurrence(mutation=None):
    """A numpy copy of the recurrence with one planted mistake (or none)."""
    def fwd(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=1.0):
        q, k, v, g, beta = (np.asarray(a, np.float64) for a in (q, k, v, g, beta))
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        flat = lambda a: a.reshape((B * T,) + a.shape[2:])
        q, k, v, g, beta = map(flat, (q, k, v, g, beta))
        cu = np.arange(B + 1) * T if cu_seqlens is None else np.asarray(cu_seqlens)
        N = len(cu) - 1
        o = np.zeros((B * T, H, dv))
        hT = np.zeros((N, H, dk, dv))
        for n in range(N):
            for h in range(H):
                S = np.zeros((dk, dv)) if h0 is None else np.array(h0[n, h], np.float64)
                for t in range(cu[n], cu[n + 1]):
                    a = 1.0 + g[t, h] if mutation == "gate_not_exp" else np.exp(g[t, h])
                    kt, vt, qt, b = k[t, h], v[t, h], q[t, h], beta[t, h]
                    if mutation == "read_before_decay":
                        p = S.T @ kt
                        S = a[:, None] * S
                    elif mutation == "decay_after_write":
                        p = S.T @ kt
                    elif mutation == "double_decay":
                        S = (a * a)[:, None] * S
                        p = S.T @ kt
                    elif mutation == "transposed_read":
                        S = a[:, None] * S
                        p = S @ kt
                    else:
                        S = a[:, None] * S
                        p = S.T @ kt
                    o_early = S.T @ qt
                    if mutation == "sign_flip":
                        S = S - b * np.outer(kt, vt - p)
                    elif mutation == "no_beta":
                        S = S + np.outer(kt, vt - p)
                    elif mutation == "beta_on_erase_only":
                        S = S + np.outer(kt, vt - b * p)
                    else:
                        S = S + b * np.outer(kt, vt - p)
                    if mutation == "decay_after_write":
                        S = a[:, None] * S
                    ot = o_early if mutation == "read_before_write" else S.T @ qt
                    o[t, h] = ot if mutation == "no_scale" else scale * ot
                hT[n, h] = S
        return o.reshape(B, T, H, dv), hT
    return fwd


MUTATIONS = ["gate_not_exp", "read_before_decay", "decay_after_write", "double_decay",
             "transposed_read", "sign_flip", "no_beta", "beta_on_erase_only",
             "read_before_write", "no_scale"]


def test_unmutated_copy_passes_all_pins():
    fwd = make_recurrence(None)
    assert all(p(fwd) for p in PINS if p is not pin_column_perm) and pin_column_perm(fwd)


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_every_planted_mistake_is_caught(mutation):
    fwd = make_recurrence(mutation)
    caught = []
    for p in PINS:
        try:
            ok = p(fwd)
        except (ValueError, np.linalg.LinAlgError):
            ok = False
        if not ok:
            caught.append(p.__name__)
    assert caught, f"no pin catches {mutation}"


def test_oracle_threads_and_heads_subset():
    """Computing a subset of heads, with any thread count, gives the same bits."""
    x = make_prefill(24, 2, 40, 4, 8, 6, in_dtype="bf16", h0_std=0.02)
    o, hT = oracle.forward(x.q, x.k, x.v, x.g, x.beta, h0=x.h0, nthreads=1)
    o2, h2 = oracle.forward(x.q, x.k, x.v, x.g, x.beta, h0=x.h0, heads=[3, 1], nthreads=3)
    assert np.array_equal(o2, o[:, :, [3, 1]]) and np.array_equal(h2, hT[:, [3, 1]])


def test_decode_step_is_one_token_prefill():
    x = make_prefill(25, 6, 1, 3, 8, 5, in_dtype="bf16", h0_std=0.02)
    o, hT = oracle.forward(x.q, x.k, x.v, x.g, x.beta, h0=x.h0)
    od, sd = oracle.decode_step(x.q[:, 0], x.k[:, 0], x.v[:, 0], x.g[:, 0], x.beta[:, 0], x.h0)
    assert np.array_equal(od, o[:, 0]) and np.array_equal(sd, hT)


def test_input_generator_recipe():
    """bf16 inputs are exact bf16 values; keys are unit norm before rounding."""
    x = make_prefill(26, 1, 64, 2, 128, 128, in_dtype="bf16")
    for a in (x.q, x.k, x.v, x.beta):
        assert np.array_equal(bf16_round(a), a)
    nk = np.linalg.norm(x.k.astype(np.float64), axis=-1)
    assert np.all(np.abs(nk - 1) < 2e-2)
    assert np.all(x.g <= 0) and np.all((x.beta > 0) & (x.beta < 1))
