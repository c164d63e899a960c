"""Independent numpy checks that pin the oracle (tests only).

`dense_delta_rule` is the closed form of the gated delta rule over a whole sequence: no recurrence,
one triangular solve (LAPACK via scipy). With H = S^T and gamma_t = sum_{i<=t} g_i, unrolling
S_t = e^{g_t} S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T gives, for the write vectors u_t,
    (I + A) U = diag(beta) V - diag(beta e^gamma) K H0,   A[r,s] = beta_r e^{gamma_r-gamma_s} k_r.k_s (s<r)
    O = scale (diag(e^gamma) Q H0 + P U),                  P[r,s] = e^{gamma_r-gamma_s} q_r.k_s (s<=r)
    H_T = e^{gamma_T} H0 + K^T diag(e^{gamma_T-gamma}) U.
`chunked_delta_rule` applies the same closed form chunk by chunk with the state carried between
chunks (the WY/UT chunk form the GPU kernels use), with the explicit inverse T = (I + A)^{-1}.
`layer` composes the whole layer from numpy/scipy primitives (np.correlate for the conv,
np.logaddexp / expit for the gates, np.repeat for the GQA head mapping).
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular
from scipy.special import expit


def l2n(x, eps):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def _decay_matrix(gam):
    """D[r, s] = exp(gamma_r - gamma_s) for s <= r, else 0 (never forms exp(gamma_r) * exp(-gamma_s))."""
    L = gam.shape[0]
    diff = gam[:, None] - gam[None, :]
    D = np.zeros((L, L))
    tril = np.tril(np.ones((L, L), dtype=bool))
    D[tril] = np.exp(diff[tril])
    return D


def dense_delta_rule_head(qn, kn, v, g, beta, H0, scale):
    """One value head, whole sequence. qn, kn [L, d_k] normalised; v [L, d_v]; H0 [d_k, d_v]."""
    L = qn.shape[0]
    gam = np.cumsum(g)
    D = _decay_matrix(gam)
    A = np.tril(beta[:, None] * D * (kn @ kn.T), -1)
    rhs = beta[:, None] * v - (beta * np.exp(gam))[:, None] * (kn @ H0)
    U = solve_triangular(np.eye(L) + A, rhs, lower=True, unit_diagonal=True)
    P = D * (qn @ kn.T)
    O = scale * (np.exp(gam)[:, None] * (qn @ H0) + P @ U)
    HT = np.exp(gam[-1]) * H0 + kn.T @ (np.exp(gam[-1] - gam)[:, None] * U)
    return O, HT


def chunked_delta_rule_head(qn, kn, v, g, beta, H0, scale, C):
    """Chunk form with the explicit UT inverse, state carried across chunks of length C."""
    L = qn.shape[0]
    H = H0.copy()
    O = np.zeros((L, v.shape[1]))
    for t0 in range(0, L, C):
        sl = slice(t0, min(t0 + C, L))
        q_, k_, v_, g_, b_ = qn[sl], kn[sl], v[sl], g[sl], beta[sl]
        n = q_.shape[0]
        gam = np.cumsum(g_)
        D = _decay_matrix(gam)
        A = np.tril(b_[:, None] * D * (k_ @ k_.T), -1)
        T = solve_triangular(np.eye(n) + A, np.eye(n), lower=True, unit_diagonal=True)
        W = T @ ((b_ * np.exp(gam))[:, None] * k_)
        Up = T @ (b_[:, None] * v_)
        U = Up - W @ H
        P = D * (q_ @ k_.T)
        O[sl] = scale * (np.exp(gam)[:, None] * (q_ @ H) + P @ U)
        H = np.exp(gam[-1]) * H + k_.T @ (np.exp(gam[-1] - gam)[:, None] * U)
    return O, H


def delta_rule(q, k, v, g, beta, H0, scale, l2_eps, C=None):
    """All heads of one sequence. q, k [L, n_k, d_k] raw; v [L, n_v, d_v]; g, beta [L, n_v];
    H0 [n_v, d_k, d_v]. Value head h reads key head h // (n_v // n_k) (np.repeat over heads)."""
    n_k, n_v = q.shape[1], v.shape[1]
    r = n_v // n_k
    qn = np.repeat(l2n(q, l2_eps), r, axis=1)
    kn = np.repeat(l2n(k, l2_eps), r, axis=1)
    O = np.zeros(v.shape)
    H = np.zeros(H0.shape)
    for h in range(n_v):
        if C is None:
            O[:, h], H[h] = dense_delta_rule_head(qn[:, h], kn[:, h], v[:, h], g[:, h], beta[:, h], H0[h], scale)
        else:
            O[:, h], H[h] = chunked_delta_rule_head(qn[:, h], kn[:, h], v[:, h], g[:, h], beta[:, h], H0[h],
                                                    scale, C)
    return O, H


def conv_silu(w, tail, x, length):
    """Per channel: np.correlate over [tail | x] (valid), then SiLU; new tail = xin[length:length+Kc]."""
    Kc = tail.shape[0]
    xin = np.concatenate([tail, x], 0)
    L, C = x.shape
    pre = np.stack([np.correlate(xin[:, c], w[c], mode="valid") for c in range(C)], axis=1)
    assert pre.shape == (L, C)
    return pre * expit(pre), xin[length:length + Kc].copy()


def gates(A_log, dt_bias, a, b, length):
    m = (np.arange(a.shape[0]) < length).astype(np.float64)[:, None]
    g = -np.exp(A_log)[None, :] * np.logaddexp(0.0, a + dt_bias[None, :]) * m
    beta = expit(b) * m
    return g, beta


def gated_rmsnorm(o, z, w, eps):
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return w * (o / rms) * (z * expit(z))


def layer(dims, weights, mixed, z, a, b, lens, tail0, H0, C=None):
    """Whole layer, B sequences, from numpy primitives. Returns (out, tail, H, o)."""
    B, L, _ = mixed.shape
    nk, nv, dk, dv = dims.n_k, dims.n_v, dims.d_k, dims.d_v
    scale = float(dk) ** -0.5 if dims.scale is None else float(dims.scale)
    f = lambda x: np.asarray(x, dtype=np.float64)
    outs, tails, Hs, os_ = [], [], [], []
    for s in range(B):
        y, tail = conv_silu(f(weights.conv_w), f(tail0[s]), f(mixed[s]), int(lens[s]))
        q = y[:, : nk * dk].reshape(L, nk, dk)
        k = y[:, nk * dk: 2 * nk * dk].reshape(L, nk, dk)
        v = y[:, 2 * nk * dk:].reshape(L, nv, dv)
        g, beta = gates(f(weights.A_log), f(weights.dt_bias), f(a[s]), f(b[s]), int(lens[s]))
        o, H = delta_rule(q, k, v, g, beta, f(H0[s]), scale, dims.l2_eps, C)
        out = gated_rmsnorm(o, f(z[s]).reshape(L, nv, dv), f(weights.norm_w), dims.rms_eps)
        outs.append(out.reshape(L, nv * dv))
        tails.append(tail)
        Hs.append(H)
        os_.append(o.reshape(L, nv * dv))
    return np.stack(outs), np.stack(tails), np.stack(Hs), np.stack(os_)
