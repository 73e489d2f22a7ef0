"""Pins for the oracle's optional input transforms (CPU only).

The pages' parameterization table puts the Q/K L2 normalization inside the KDA
kernel, and their list of the public tests names a fused gate.  The oracle
applies both, per token and in fp64, before the recurrence:

* qk_l2norm: x / sqrt(sum x^2 + eps), eps = 1e-6 (the pages give no eps);
* gate_logits: the log-gate is -gate_scale * softplus(z) for logits z.

They are pinned here against facts that hold without the oracle:

* a one-token example worked by hand (3-4-5 vectors);
* invariance to a positive per-token rescaling of q and of k;
* rows that are already exactly unit-norm (Hadamard rows) pass unchanged;
* the gate equals the log-gate formed with numpy's logaddexp (log(e^0 + e^z));
* closed forms: z = 0 gives alpha = 2^-gate_scale, z -> -inf gives alpha = 1;
* a scalar gate per token and head (g of shape [B, T, H]) is Gated DeltaNet:
  the separately written numpy Gated DeltaNet gives the same result.

Deliberately wrong transforms (planted on the CPU) show that each pin set
catches the plausible mistakes.
"""
import numpy as np
import pytest

import oracle
from oracle import reference as ref
from gated_delta_rule_52_amd.inputs import make_prefill
from test_oracle import hadamard_keys, rel


def oracle_fwd(q, k, v, g, beta, h0=None, cu_seqlens=None, **tr):
    return oracle.forward(q, k, v, g, beta, h0=h0, cu_seqlens=cu_seqlens, **tr)


def case(seed, T=11, H=2, dk=8, dv=5):
    return make_prefill(seed, 1, T, H, dk, dv, in_dtype="fp32", h0_std=0.5, fused=True)


def run(fwd, x, q=None, k=None, g=None, **tr):
    return fwd(x.q if q is None else q, x.k if k is None else k, x.v, x.g if g is None else g, x.beta,
               h0=x.h0, cu_seqlens=x.cu_seqlens, **tr)


# --------------------------------------------------------------------- L2 norm

def pin_l2_worked_example(fwd):
    """One token, zero state, alpha = 1, beta = 1: S_1 = k^ v^T and o = (k^.q^) v.
    q = (3, 4, 0, 0) and k = (4, 3, 0, 0) normalise to (0.6, 0.8, 0, 0) and
    (0.8, 0.6, 0, 0), so o = 0.96 v and the state rows are 0.8 v, 0.6 v, 0, 0."""
    f = np.float32
    q = np.array([3, 4, 0, 0], f).reshape(1, 1, 1, 4)
    k = np.array([4, 3, 0, 0], f).reshape(1, 1, 1, 4)
    v = np.array([1.0, -2.0], f).reshape(1, 1, 1, 2)
    g = np.zeros((1, 1, 1, 4), f)
    beta = np.ones((1, 1, 1), f)
    o, hT = fwd(q, k, v, g, beta, qk_l2norm=True, gate_logits=False, gate_scale=1.0)
    want_o = 0.96 * v.reshape(2).astype(np.float64)
    want_s = np.outer([0.8, 0.6, 0.0, 0.0], v.reshape(2))
    return rel(o.reshape(2), want_o) < 1e-7 and rel(hT.reshape(4, 2), want_s) < 1e-7


def pin_l2_scale_invariance(fwd):
    """Rescaling each token's q and k by positive factors changes nothing
    (up to the eps term, below 1e-6 relative for these norms)."""
    x = case(90)
    rng = np.random.default_rng(91)
    cq = rng.uniform(0.5, 4.0, size=x.q.shape[:3] + (1,)).astype(np.float32)
    ck = rng.uniform(0.5, 4.0, size=x.k.shape[:3] + (1,)).astype(np.float32)
    tr = dict(qk_l2norm=True, gate_logits=True, gate_scale=1.0)
    o1, h1 = run(fwd, x, **tr)
    o2, h2 = run(fwd, x, q=x.q * cq, **tr)
    o3, h3 = run(fwd, x, k=x.k * ck, **tr)
    return max(rel(o2, o1), rel(h2, h1), rel(o3, o1), rel(h3, h1)) < 1e-5


def pin_l2_unit_rows_unchanged(fwd):
    """Exactly unit-norm rows (entries +-1/4 of a 16-wide Hadamard matrix)
    give the result without the transform, to the eps term (5e-7)."""
    x = case(92, T=9, H=1, dk=16, dv=4)
    kh = hadamard_keys(16, 9, 93).reshape(1, 9, 1, 16)
    qh = hadamard_keys(16, 9, 94).reshape(1, 9, 1, 16)
    on = run(fwd, x, q=qh, k=kh, qk_l2norm=True, gate_logits=True, gate_scale=1.0)
    off = run(fwd, x, q=qh, k=kh, qk_l2norm=False, gate_logits=True, gate_scale=1.0)
    return rel(on[0], off[0]) < 2e-6 and rel(on[1], off[1]) < 2e-6


# ------------------------------------------------------------------------ gate

def pin_gate_logaddexp(fwd):
    """The gate from logits equals the log-gate -s * logaddexp(0, z) handed
    over directly (numpy's routine; g rounds to float32 on the way)."""
    x = case(95)
    s = 0.7
    g = (-s * np.logaddexp(0.0, x.g.astype(np.float64))).astype(np.float32)
    a = run(fwd, x, qk_l2norm=True, gate_logits=True, gate_scale=s)
    b = run(fwd, x, g=g, qk_l2norm=True, gate_logits=False, gate_scale=1.0)
    return rel(a[0], b[0]) < 1e-6 and rel(a[1], b[1]) < 1e-6


def pin_gate_closed_forms(fwd):
    """z = 0: alpha = 2^-s, i.e. g = -s ln 2; z = -60: alpha = 1 to e^-60."""
    x = case(96)
    s = 1.3
    zero, very_neg = np.zeros_like(x.g), np.full_like(x.g, -60.0)
    a = run(fwd, x, g=zero, qk_l2norm=True, gate_logits=True, gate_scale=s)
    b = run(fwd, x, g=np.full_like(x.g, -s * np.log(2.0)), qk_l2norm=True, gate_logits=False, gate_scale=1.0)
    c = run(fwd, x, g=very_neg, qk_l2norm=True, gate_logits=True, gate_scale=s)
    d = run(fwd, x, g=np.zeros_like(x.g), qk_l2norm=True, gate_logits=False, gate_scale=1.0)
    return (rel(a[0], b[0]) < 1e-6 and rel(a[1], b[1]) < 1e-6
            and rel(c[0], d[0]) < 1e-12 and rel(c[1], d[1]) < 1e-12)


def pin_scalar_gate_is_gdn(fwd):
    """One gate per token and head, for every key channel: the recurrence is
    Gated DeltaNet, S_t = alpha_t (I - beta k k^T) S + beta k v^T (independent
    numpy form), with alpha = exp(g), or exp(-s softplus(z)) from logits."""
    x = make_prefill(98, 1, 13, 2, 6, 4, in_dtype="fp32", h0_std=0.5, scalar_gate=True)
    ok = True
    for logits, s in ((False, 1.0), (True, 0.6)):
        g = x.g.astype(np.float64)
        lg = -s * np.logaddexp(0.0, g) if logits else g
        o, hT = fwd(x.q, x.k, x.v, x.g, x.beta, h0=x.h0, qk_l2norm=False, gate_logits=logits,
                    gate_scale=s, scalar_gate=True)
        o2, S2 = ref.gated_deltanet(x.q[0], x.k[0], x.v[0], np.exp(lg[0]), x.beta[0], x.h0[0])
        # 1e-6: a harness that forms the log-gate itself hands it over in float32
        ok = ok and max(rel(o[0], o2), rel(hT[0], S2)) < (1e-6 if logits else 1e-12)
    return ok


PINS = [pin_l2_worked_example, pin_l2_scale_invariance, pin_l2_unit_rows_unchanged,
        pin_gate_logaddexp, pin_gate_closed_forms, pin_scalar_gate_is_gdn]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_transform_pin(pin):
    assert pin(oracle_fwd)


# -------------------------------------------- planted mistakes (CPU, numpy)

def make_transformed(mutation=None):
    """Apply the transforms in numpy (one planted mistake, or none), then the
    oracle with both switched off."""
    def fwd(q, k, v, g, beta, h0=None, cu_seqlens=None, qk_l2norm=False, gate_logits=False, gate_scale=1.0,
            scalar_gate=False):
        q, k, g = (np.asarray(a, np.float64) for a in (q, k, g))
        if scalar_gate:  # one gate per token and head, for every key channel
            g = np.repeat(g[..., None], q.shape[-1], axis=-1)
            if mutation == "scalar_gate_first_channel":
                g[..., 1:] = -60.0 if gate_logits else 0.0
        if qk_l2norm:
            def nrm(x):
                if mutation == "l2_no_sqrt":
                    return x / ((x * x).sum(-1, keepdims=True) + 1e-6)
                if mutation == "l2_l1":
                    return x / np.abs(x).sum(-1, keepdims=True)
                return x / np.sqrt((x * x).sum(-1, keepdims=True) + 1e-6)
            q = q if mutation == "l2_k_only" else nrm(q)
            k = k if mutation == "l2_q_only" else nrm(k)
        if gate_logits:
            s = 1.0 if mutation == "gate_no_scale" else gate_scale
            sp = {"gate_exp": np.exp(g), "gate_log_only": g, "gate_relu": np.maximum(g, 0.0)}.get(
                mutation, np.logaddexp(0.0, g))
            g = s * sp if mutation == "gate_plus" else -s * sp
        return oracle.forward(q.astype(np.float32), k.astype(np.float32), v, g.astype(np.float32), beta,
                              h0=h0, cu_seqlens=cu_seqlens)
    return fwd


MUTATIONS = ["l2_no_sqrt", "l2_l1", "l2_q_only", "l2_k_only", "gate_plus", "gate_no_scale",
             "gate_exp", "gate_log_only", "gate_relu", "scalar_gate_first_channel"]


def test_numpy_transform_passes_all_pins():
    fwd = make_transformed(None)
    assert all(p(fwd) for p in PINS)


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_every_planted_transform_mistake_is_caught(mutation):
    fwd = make_transformed(mutation)
    caught = []
    for p in PINS:
        with np.errstate(all="ignore"):
            ok = p(fwd)
        if not ok:
            caught.append(p.__name__)
    assert caught, f"no pin catches {mutation}"


def test_decode_step_takes_the_transforms():
    """A decode step with the transforms is the one-token prefill with them."""
    x = make_prefill(97, 5, 1, 3, 8, 6, in_dtype="bf16", h0_std=0.02, fused=True)
    tr = x.transforms()
    o, hT = oracle.forward(x.q, x.k, x.v, x.g, x.beta, h0=x.h0, **tr)
    od, sd = oracle.decode_step(x.q[:, 0], x.k[:, 0], x.v[:, 0], x.g[:, 0], x.beta[:, 0], x.h0, **tr)
    assert np.array_equal(od, o[:, 0]) and np.array_equal(sd, hT)
