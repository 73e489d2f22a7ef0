"""Independent fp64 numpy references used to pin the oracle.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).

Each function is written on its own, in a form textually different from the
C recurrence in ``kda_oracle.c``, so that a mistake in one does not repeat in
the other.  All take one sequence: q, k, g are [T, H, dk], v is [T, H, dv],
beta is [T, H], S0 is [H, dk, dv] (or None).  They return (o [T, H, dv],
S_T [H, dk, dv]) in float64.

Sources (the pages on Kimi Linear):
* research-notes-dl6 review notes, section "Method / from Linear Attention to
  KDA": vanilla linear attention, the DeltaNet update and its read-then-write
  form, the KDA recurrence with per-channel Diag(alpha);
* same page, "Mathematical Rigor", issue 3: the corrected cumulative decay
  gamma^{i->j} = prod_{k=i+1..j} alpha^k, gamma^r = prod_{k=1..r} alpha^k;
* jxzklqfsx.com article, section on the hardware-efficient chunkwise
  algorithm: WY representation, UT transform, row-wise forward substitution,
  inter-chunk recurrence with intra-chunk parallel output (its formulas are
  missing from the page; the chunk form below is derived from the recurrence
  and pinned against it by chunk-size invariance).
"""
from __future__ import annotations

import numpy as np

f64 = np.float64


def _prep(q, k, v, g, beta, S0):
    q, k, v, g, beta = (np.asarray(x, dtype=f64) for x in (q, k, v, g, beta))
    T, H, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((H, dk, dv)) if S0 is None else np.array(S0, dtype=f64)
    return q, k, v, g, beta, S, T, H, dk, dv


def kda_dense_transition(q, k, v, g, beta, S0=None, scale=1.0):
    """Brute force with explicit dk x dk transitions.

    S_t = M_t S_{t-1} + beta_t k_t v_t^T with M_t = (I - beta_t k_t k_t^T) Diag(alpha_t),
    the KDA recurrence in its first (product) form; o_t = scale S_t^T q_t.
    """
    q, k, v, g, beta, S, T, H, dk, dv = _prep(q, k, v, g, beta, S0)
    o = np.zeros((T, H, dv))
    eye = np.eye(dk)
    for h in range(H):
        for t in range(T):
            kt = k[t, h][:, None]
            M = (eye - beta[t, h] * (kt @ kt.T)) @ np.diag(np.exp(g[t, h]))
            S[h] = M @ S[h] + beta[t, h] * (kt @ v[t, h][None, :])
            o[t, h] = scale * (S[h].T @ q[t, h])
    return o, S


def linear_attention(q, k, v):
    """Vanilla linear attention written as a causal sum, no state:
    o_t = sum_{i<=t} (k_i . q_t) v_i, which is S_t^T q_t for S_t = sum_{i<=t} k_i v_i^T."""
    q, k, v = (np.asarray(x, dtype=f64) for x in (q, k, v))
    T, H, _ = k.shape
    o = np.zeros((T, H, v.shape[-1]))
    for h in range(H):
        scores = q[:, h] @ k[:, h].T          # [T, T]: (t, i) -> q_t . k_i
        o[:, h] = np.tril(scores) @ v[:, h]
    return o


def deltanet(q, k, v, beta, S0=None):
    """DeltaNet in its read-then-write-residual form (no decay):
    S_t = S_{t-1} + beta_t k_t (v_t - S_{t-1}^T k_t)^T, o_t = S_t^T q_t."""
    T, H, dk = np.shape(k)
    g0 = np.zeros((T, H, dk))
    q, k, v, _, beta, S, T, H, dk, dv = _prep(q, k, v, g0, beta, S0)
    o = np.zeros((T, H, dv))
    for t in range(T):
        for h in range(H):
            resid = v[t, h] - np.einsum("ij,i->j", S[h], k[t, h])
            S[h] += beta[t, h] * np.outer(k[t, h], resid)
            o[t, h] = np.einsum("ij,i->j", S[h], q[t, h])
    return o, S


def gated_deltanet(q, k, v, alpha, beta, S0=None):
    """Gated DeltaNet with one scalar forget rate per token and head:
    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t."""
    T, H, dk = np.shape(k)
    g0 = np.zeros((T, H, dk))
    q, k, v, _, beta, S, T, H, dk, dv = _prep(q, k, v, g0, beta, S0)
    alpha = np.asarray(alpha, dtype=f64)
    o = np.zeros((T, H, dv))
    for t in range(T):
        for h in range(H):
            kk = np.outer(k[t, h], k[t, h])
            S[h] = alpha[t, h] * (S[h] - beta[t, h] * kk @ S[h]) + beta[t, h] * np.outer(k[t, h], v[t, h])
            o[t, h] = S[h].T @ q[t, h]
    return o, S


def decay_only(q, g, S0, scale=1.0):
    """beta = 0: nothing is written, so S_t = Diag(exp(sum_{s<=t} g_s)) S_0 in closed form."""
    q, g, S0 = (np.asarray(x, dtype=f64) for x in (q, g, S0))
    G = np.cumsum(g, axis=0)                  # [T, H, dk]
    St = np.exp(G)[..., None] * S0[None]      # [T, H, dk, dv]
    o = scale * np.einsum("thij,thi->thj", St, q)
    return o, St[-1]


def kda_chunked(q, k, v, g, beta, S0=None, scale=1.0, C=64):
    """fp64 chunkwise form with chunk size C (the last chunk may be shorter).

    Per chunk with rows r = 1..L and entering state S:
      G_r   = g_1 + ... + g_r (chunk-local, inclusive), so gamma^{i->r} = exp(G_r - G_i)
      A_kk[r,i] = beta_r sum_c k_r[c] k_i[c] exp(G_r[c] - G_i[c])          (i < r)
      A_qk[r,i] = scale sum_c q_r[c] k_i[c] exp(G_r[c] - G_i[c])           (i <= r)
      T_ut  = (I + A_kk)^{-1}, by forward substitution one row at a time
      W = T_ut (beta * exp(G) * K),  U = T_ut (beta * V)                   (WY factors)
      V_new = U - W S
      O     = scale (exp(G) * Q) S + A_qk V_new                           (inter + intra)
      S    <- exp(G_L) * S + (exp(G_L - G) * K)^T V_new                   (next state)
    """
    q, k, v, g, beta, S, T, H, dk, dv = _prep(q, k, v, g, beta, S0)
    o = np.zeros((T, H, dv))
    for h in range(H):
        Sh = S[h]
        for c0 in range(0, T, C):
            c1 = min(T, c0 + C)
            L = c1 - c0
            Q, K, V = q[c0:c1, h], k[c0:c1, h], v[c0:c1, h]
            b = beta[c0:c1, h]
            G = np.cumsum(g[c0:c1, h], axis=0)                       # [L, dk]
            D = np.exp(G[:, None, :] - G[None, :, :])                  # [r, i, c]
            Akk = np.zeros((L, L))
            Aqk = np.zeros((L, L))
            for r in range(L):
                for i in range(r + 1):
                    if i < r:
                        Akk[r, i] = b[r] * np.sum(K[r] * K[i] * D[r, i])
                    Aqk[r, i] = scale * np.sum(Q[r] * K[i] * D[r, i])
            # forward substitution: T[r,:] = e_r - sum_{i<r} Akk[r,i] T[i,:]
            Tut = np.zeros((L, L))
            for r in range(L):
                Tut[r, r] = 1.0
                for i in range(r):
                    Tut[r, :] -= Akk[r, i] * Tut[i, :]
            W = Tut @ (b[:, None] * np.exp(G) * K)
            U = Tut @ (b[:, None] * V)
            Vn = U - W @ Sh
            o[c0:c1, h] = scale * (np.exp(G) * Q) @ Sh + Aqk @ Vn
            Sh = np.exp(G[-1])[:, None] * Sh + (np.exp(G[-1][None, :] - G) * K).T @ Vn
        S[h] = Sh
    return o, S
