"""Pins for the oracle's gradients (CPU only).

The backward is checked against the definition of a derivative and against
closed forms, never against itself:

* central finite differences of the fp64 forward, Richardson-extrapolated
  (error O(eps^4)), for every element of every input on a tiny problem.  The
  forward takes float32 inputs, so inputs sit on a 2^-12 grid and the
  perturbations are +-2^-7 and +-2^-8: every perturbed value is exact;
* alpha = 1 and beta = 0: the state never changes, so o_t = scale S_0^T q_t and
  every gradient has a short closed form;
* one token from a zero state: o = scale beta (k.q) v and S_1 = beta k v^T.

The loss is L = sum(o * W) + sum(S_T * Wh), so the output gradient is W and
the final-state gradient is Wh.
"""
import numpy as np
import pytest

import oracle


def grid(rng, shape, lo, hi):
    """Uniform values rounded to multiples of 2^-12 (exact in float32)."""
    return (np.round(rng.uniform(lo, hi, size=shape) * 4096) / 4096).astype(np.float32)


def tiny(seed, T=4, H=1, dk=3, dv=2, N=1):
    rng = np.random.default_rng(seed)
    x = dict(q=grid(rng, (N, T, H, dk), -1, 1), k=grid(rng, (N, T, H, dk), -1, 1),
             v=grid(rng, (N, T, H, dv), -1, 1), g=grid(rng, (N, T, H, dk), -0.7, -0.05),
             beta=grid(rng, (N, T, H), 0.1, 0.9))
    h0 = grid(rng, (N, H, dk, dv), -0.5, 0.5).astype(np.float64)
    W = rng.standard_normal((N, T, H, dv))
    Wh = rng.standard_normal((N, H, dk, dv))
    return x, h0, W, Wh


def loss(x, h0, W, Wh, scale, scalar_gate=False, **tr):
    o, hT = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=h0, scale=scale, scalar_gate=scalar_gate,
                           **tr)
    return float(np.sum(o * W) + np.sum(hT * Wh))


def fd_gradient(x, h0, W, Wh, scale, name, idx, scalar_gate=False, **tr):
    def shifted(eps):
        if name == "h0":
            hp, hm = h0.copy(), h0.copy()
            hp[idx] += eps
            hm[idx] -= eps
            return (loss(x, hp, W, Wh, scale, scalar_gate, **tr) - loss(x, hm, W, Wh, scale, scalar_gate, **tr)) / (2 * eps)
        xp = {k: a.copy() for k, a in x.items()}
        xm = {k: a.copy() for k, a in x.items()}
        xp[name][idx] += np.float32(eps)
        xm[name][idx] -= np.float32(eps)
        return (loss(xp, h0, W, Wh, scale, scalar_gate, **tr) - loss(xm, h0, W, Wh, scale, scalar_gate, **tr)) / (2 * eps)
    d1, d2 = shifted(2.0 ** -7), shifted(2.0 ** -8)
    return (4 * d2 - d1) / 3


@pytest.mark.parametrize("scale", [1.0, 0.7])
def test_backward_matches_finite_differences(scale):
    x, h0, W, Wh = tiny(130)
    r = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], W.astype(np.float32), h0=h0,
                        d_final_state=Wh, scale=scale)
    W32 = W.astype(np.float32).astype(np.float64)  # the output gradient the oracle sees
    key = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "h0": "dh0"}
    for name, arr in list(x.items()) + [("h0", h0)]:
        fd = np.zeros(arr.shape)
        for idx in np.ndindex(arr.shape):
            fd[idx] = fd_gradient(x, h0, W32, Wh, scale, name, idx)
        an = r[key[name]]
        err = np.linalg.norm(an - fd) / max(np.linalg.norm(fd), 1e-30)
        assert err < 1e-8, (name, err)


def test_backward_scalar_gate_matches_finite_differences():
    """One gate per token and head (Gated DeltaNet): every element of every
    input against Richardson-extrapolated central differences."""
    x, h0, W, Wh = tiny(133)
    rng = np.random.default_rng(134)
    x["g"] = grid(rng, x["beta"].shape, -0.7, -0.05)  # [N, T, H]
    r = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], W.astype(np.float32), h0=h0,
                        d_final_state=Wh, scale=0.9, scalar_gate=True)
    W32 = W.astype(np.float32).astype(np.float64)
    key = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "h0": "dh0"}
    for name, arr in list(x.items()) + [("h0", h0)]:
        fd = np.zeros(arr.shape)
        for idx in np.ndindex(arr.shape):
            fd[idx] = fd_gradient(x, h0, W32, Wh, 0.9, name, idx, scalar_gate=True)
        an = r[key[name]]
        assert an.shape == fd.shape, (name, an.shape, fd.shape)
        err = np.linalg.norm(an - fd) / max(np.linalg.norm(fd), 1e-30)
        assert err < 1e-8, (name, err)


@pytest.mark.parametrize("scalar_gate", [False, True], ids=["channel_gate", "scalar_gate"])
def test_backward_with_transforms_matches_finite_differences(scalar_gate):
    """The L2 norm of q and k and the softplus gate from logits (gate scale
    0.8): gradients of the raw inputs against central differences of the
    forward with the same transforms."""
    x, h0, W, Wh = tiny(135)
    rng = np.random.default_rng(136)
    x["q"] = grid(rng, x["q"].shape, -2, 2)
    x["k"] = grid(rng, x["k"].shape, -2, 2)
    x["g"] = grid(rng, x["beta"].shape if scalar_gate else x["g"].shape, -2, 2)  # logits
    tr = dict(qk_l2norm=True, gate_logits=True, gate_scale=0.8)
    r = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], W.astype(np.float32), h0=h0,
                        d_final_state=Wh, scale=1.1, scalar_gate=scalar_gate, **tr)
    W32 = W.astype(np.float32).astype(np.float64)
    key = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "h0": "dh0"}
    for name, arr in list(x.items()) + [("h0", h0)]:
        fd = np.zeros(arr.shape)
        for idx in np.ndindex(arr.shape):
            fd[idx] = fd_gradient(x, h0, W32, Wh, 1.1, name, idx, scalar_gate=scalar_gate, **tr)
        err = np.linalg.norm(r[key[name]] - fd) / max(np.linalg.norm(fd), 1e-30)
        assert err < 1e-7, (name, err)


def test_backward_frozen_state_closed_form():
    """alpha = 1, beta = 0: S_t = S_0, o_t = s S_0^T q_t.  With dS_t =
    Wh + s sum_{r >= t} q_r W_r^T and u_t = v_t - S_0^T k_t:
    dq_t = s S_0 W_t, dk_t = -S_0 (beta dS_t^T k_t) = 0, dv_t = 0,
    dbeta_t = k_t^T dS_t u_t, dg_t = rowsum(S_0 . dS_t), dh0 = dS_1."""
    rng = np.random.default_rng(131)
    N, T, H, dk, dv, s = 1, 6, 2, 5, 3, 0.8
    q, k, v = (rng.standard_normal((N, T, H, d)).astype(np.float32) for d in (dk, dk, dv))
    g = np.zeros((N, T, H, dk), np.float32)
    beta = np.zeros((N, T, H), np.float32)
    h0 = rng.standard_normal((N, H, dk, dv))
    W = rng.standard_normal((N, T, H, dv)).astype(np.float32)
    Wh = rng.standard_normal((N, H, dk, dv))
    r = oracle.backward(q, k, v, g, beta, W, h0=h0, d_final_state=Wh, scale=s)
    for h in range(H):
        S0 = h0[0, h]
        dS = Wh[0, h].copy()
        for t in range(T - 1, -1, -1):
            qt, kt, vt, wt = (a[0, t, h].astype(np.float64) for a in (q, k, v, W))
            dS = dS + s * np.outer(qt, wt)
            assert np.allclose(r["dq"][0, t, h], s * S0 @ wt, rtol=1e-12, atol=1e-12)
            assert np.allclose(r["dk"][0, t, h], 0.0, atol=1e-12)
            assert np.allclose(r["dv"][0, t, h], 0.0, atol=1e-12)
            u = vt - S0.T @ kt
            assert np.isclose(r["dbeta"][0, t, h], kt @ dS @ u, rtol=1e-12, atol=1e-12)
            assert np.allclose(r["dg"][0, t, h], np.sum(S0 * dS, axis=1), rtol=1e-12, atol=1e-12)
        assert np.allclose(r["dh0"][0, h], dS, rtol=1e-12, atol=1e-12)


def test_backward_one_token_closed_form():
    """One token from a zero state: o = s b (k.q) v, S_1 = b k v^T."""
    rng = np.random.default_rng(132)
    dk, dv, s = 4, 3, 1.3
    q, k = (rng.standard_normal((1, 1, 1, dk)).astype(np.float32) for _ in range(2))
    v = rng.standard_normal((1, 1, 1, dv)).astype(np.float32)
    g = -np.abs(rng.standard_normal((1, 1, 1, dk))).astype(np.float32)
    beta = np.array([[[0.6]]], np.float32)
    W = rng.standard_normal((1, 1, 1, dv)).astype(np.float32)
    Wh = rng.standard_normal((1, 1, dk, dv))
    r = oracle.backward(q, k, v, g, beta, W, h0=None, d_final_state=Wh, scale=s)
    qv, kv, vv, wv = (a.reshape(-1).astype(np.float64) for a in (q, k, v, W))
    b = float(beta.reshape(-1)[0])  # the float32 value the oracle sees
    al = np.exp(g.reshape(-1).astype(np.float64))
    kq, vw = kv @ qv, vv @ wv
    assert np.allclose(r["dq"].reshape(-1), s * b * vw * kv, rtol=1e-12)
    assert np.allclose(r["dk"].reshape(-1), s * b * vw * qv + b * Wh[0, 0] @ vv, rtol=1e-12)
    assert np.allclose(r["dv"].reshape(-1), s * b * kq * wv + b * Wh[0, 0].T @ kv, rtol=1e-12)
    assert np.isclose(r["dbeta"].reshape(-1)[0], s * kq * vw + kv @ Wh[0, 0] @ vv, rtol=1e-12)
    assert np.allclose(r["dg"], 0.0, atol=1e-15)  # S~ = 0
    dS = Wh[0, 0] + s * np.outer(qv, wv)
    du = b * dS.T @ kv
    assert np.allclose(r["dh0"][0, 0], al[:, None] * (dS - np.outer(kv, du)), rtol=1e-12)
