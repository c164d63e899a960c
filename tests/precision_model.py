"""Rounding model of the chunked prefill's MFMA operands (numpy, CPU). TEST INFRASTRUCTURE ONLY.

The prefill kernels run the chunk form of the gated delta rule on f16 MFMA with fp32 accumulation. Each
operand is either a single f16 value or a hi/lo pair of f16 values (hi = f16(x), lo = f16(x - hi): about
22 bits), carried multiplied by an exact power of two so that MFMA's flush of f16 subnormals (|y| < 2^-14)
does not eat small entries. This module runs the same chunk form in fp64 with every operand rounded the
way a kernel rounds it, so the error each choice costs can be read off against the layer's bounds (2e-3
on outputs, 1e-3 of max |H| on states) without a GPU. Accumulation is exact here: fp32 accumulation adds
about 2^-24 per step, far below the operands' rounding.

Chunk form (chunk of C tokens, gamma the in-chunk cumulative log decay, H = S^T the state):
  A[r][s] = beta_r e^{gamma_r - gamma_s} k_r.k_s (s < r),   P[t][s] = scale e^{gamma_t - gamma_s} q_t.k_s (s <= t)
  U = (I + A)^{-1} diag(beta) (V - diag(e^gamma) K H)
  O = scale diag(e^gamma) Q H + P U,    H <- e^{gamma_C} H + K^T diag(e^{gamma_C - gamma}) U
Two arrangements of the same algebra are modelled:
  "fused"     (the fused kernel): U by blocked substitution over 16-token blocks, U_m = T_mm (Y_m -
              sum_{j<m} A_mj U_j), T_mm = (I + A_mm)^{-1}; K H with K single;
  "two_phase" (chunk_prep + state pass): U = U' - W H with W = T diag(beta e^gamma) K and
              U' = T diag(beta) V, T = (I + A)^{-1} rounded to a single f16, W a single f16.
A configuration maps each operand to "x" (exact), "h" (single f16) or "s" (hi/lo pair), and each operand
has its power-of-two scale.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular

F16_MIN_NORMAL = 2.0 ** -14


def f16(y):
    """Round to f16 (ties to even) as MFMA reads it: subnormal results flushed to zero."""
    h = np.asarray(y, np.float32).astype(np.float16).astype(np.float64)
    return np.where(np.abs(h) < F16_MIN_NORMAL, 0.0, h)


def operand(x, mode, scale):
    """x carried as `mode` ("x", "h", "s") at the power-of-two `scale`, returned unscaled."""
    if mode == "x":
        return np.asarray(x, np.float64)
    xs = np.asarray(np.asarray(x, np.float64) * scale, np.float32).astype(np.float64)  # one fp32 value
    hi = f16(xs)
    if mode == "h":
        return hi / scale
    return (hi + f16(xs - hi)) / scale


def decay_matrix(gam):
    """D[r][s] = e^{gamma_r - gamma_s} for s <= r, else 0 (never e^{gamma_r} e^{-gamma_s})."""
    L = gam.shape[0]
    D = np.zeros((L, L))
    tri = np.tril(np.ones((L, L), dtype=bool))
    D[tri] = np.exp((gam[:, None] - gam[None, :])[tri])
    return D


# the operand choices of the two kernels for bf16 activations, and their scales
FUSED = dict(form="fused", gram="s", kh="h", H="s", A="h", Tmm="s", Z="s", U="s", Q="s", P="s", Kt="s")
TWO_PHASE = dict(form="two_phase", gram="s", T="h", X="h", V="s", W="h", H="s", U="s", Q="s", P="s", Kt="s",
                 q_folded=True)
SCALES = dict(gram=256.0, kh=256.0, H=256.0, A=256.0, Tmm=256.0, Z=256.0, U=256.0, Q=256.0, P=65536.0, Kt=256.0,
              T=256.0, X=256.0, V=256.0, W=1.0)
# the two-phase record: Q~ and P~ (scale and decays folded in) at 2^16, -W at 2^8
TWO_PHASE_SCALES = dict(SCALES, P=65536.0, Q=65536.0, W=256.0)


def all_exact(form):
    base = FUSED if form == "fused" else TWO_PHASE
    return {k: (v if k in ("form", "q_folded") else "x") for k, v in base.items()}


def head(q, k, v, g, beta, H0, scale, cfg, scales=SCALES, C=64):
    """One value head over a whole sequence: q, k [L, d_k] normalised, v [L, d_v], g, beta [L]."""
    def R(x, name):
        return operand(x, cfg[name], scales[name])

    L = q.shape[0]
    H = np.asarray(H0, np.float64).copy()
    O = np.zeros((L, v.shape[1]))
    for t0 in range(0, L, C):
        sl = slice(t0, min(t0 + C, L))
        q_, k_, v_, g_, b_ = q[sl], k[sl], v[sl], g[sl], beta[sl]
        n = q_.shape[0]
        gam = np.cumsum(g_)
        Dm = decay_matrix(gam)
        kg, qg = R(k_, "gram"), R(q_, "gram")
        A = np.tril(b_[:, None] * Dm * (kg @ kg.T), -1)
        P = scale * Dm * (qg @ kg.T)
        Hh = R(H, "H")
        if cfg["form"] == "fused":
            Y = b_[:, None] * (v_ - np.exp(gam)[:, None] * (R(k_, "kh") @ Hh))
            U = np.zeros_like(Y)
            for m0 in range(0, n, 16):
                m1 = min(m0 + 16, n)
                Z = Y[m0:m1].copy()
                for j0 in range(0, m0, 16):
                    Z -= R(A[m0:m1, j0:j0 + 16], "A") @ R(U[j0:j0 + 16], "U")
                Tmm = solve_triangular(np.eye(m1 - m0) + A[m0:m1, m0:m1], np.eye(m1 - m0), lower=True,
                                       unit_diagonal=True)
                U[m0:m1] = R(Tmm, "Tmm") @ R(Z, "Z")
        else:
            T = solve_triangular(np.eye(n) + A, np.eye(n), lower=True, unit_diagonal=True)
            Tr = R(T, "T")
            W = Tr @ R((b_ * np.exp(gam))[:, None] * k_, "X")
            Up = Tr @ R(b_[:, None] * v_, "V")
            U = Up - R(W, "W") @ Hh
        Ur = R(U, "U")
        qe = scale * np.exp(gam)[:, None]
        if cfg.get("q_folded"):
            O[sl] = R(qe * q_, "Q") @ Hh + R(P, "P") @ Ur
        else:
            O[sl] = qe * (R(q_, "Q") @ Hh) + R(P, "P") @ Ur
        H = np.exp(gam[-1]) * H + R(np.exp(gam[-1] - gam)[:, None] * k_, "Kt").T @ Ur
    return O, H


def layer_core(qn, kn, v, g, beta, H0, scale, cfg, scales=SCALES):
    """All value heads of one sequence: qn, kn [L, n_k, d_k] normalised; v [L, n_v, d_v]; value head h reads
    key head h // (n_v // n_k). Returns (o [L, n_v, d_v], H [n_v, d_k, d_v])."""
    nk, nv = qn.shape[1], v.shape[1]
    r = nv // nk
    outs, Hs = [], []
    for h in range(nv):
        O, H = head(qn[:, h // r], kn[:, h // r], v[:, h], g[:, h], beta[:, h], H0[h], scale, cfg, scales)
        outs.append(O)
        Hs.append(H)
    return np.stack(outs, 1), np.stack(Hs)


def gated_rmsnorm(o, z, w, eps):
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return w * (o / rms) * (z / (1.0 + np.exp(-z)))


def layer_inputs(seed, dims, L, n_heads, h0_std):
    """The chunk form's inputs for the first `n_heads` value heads of one sequence of the seeded layer:
    conv + SiLU and the gates in fp64 from the generated bf16 values, q and k L2-normalised."""
    import gdn_inputs
    from tests import bruteforce as bf

    w, x, rng = gdn_inputs.make_layer(seed, dims, 1, L)
    f = lambda a: np.asarray(a, np.float64)
    nk, nv, dk, dv = dims.n_k, dims.n_v, dims.d_k, dims.d_v
    r = nv // nk
    n_keys = -(-n_heads // r)
    cols = np.r_[0:n_keys * dk, nk * dk:(nk + n_keys) * dk, 2 * nk * dk:2 * nk * dk + n_heads * dv]
    y, _ = bf.conv_silu(f(w.conv_w)[cols], np.zeros((dims.kc, cols.size)), f(x.mixed[0])[:, cols], L)
    q = bf.l2n(y[:, :n_keys * dk].reshape(L, n_keys, dk), dims.l2_eps)
    k = bf.l2n(y[:, n_keys * dk:2 * n_keys * dk].reshape(L, n_keys, dk), dims.l2_eps)
    v = y[:, 2 * n_keys * dk:].reshape(L, n_heads, dv)
    g, beta = bf.gates(f(w.A_log)[:n_heads], f(w.dt_bias)[:n_heads], f(x.a[0])[:, :n_heads],
                       f(x.b[0])[:, :n_heads], L)
    H0 = rng.standard_normal((n_heads, dk, dv)) * h0_std
    z = f(x.z[0]).reshape(L, nv, dv)[:, :n_heads]
    return dict(q=q, k=k, v=v, g=g, beta=beta, H0=H0, z=z, norm_w=f(w.norm_w), scale=dims.q_scale,
                rms_eps=dims.rms_eps, r=r)


def run(inp, cfg, scales=SCALES):
    """(gated-norm output [L, n_heads, d_v], final H [n_heads, d_k, d_v]) under the configuration."""
    from threadpoolctl import threadpool_limits

    L, nh = inp["v"].shape[:2]
    outs, Hs = [], []
    with threadpool_limits(1):  # products of 64-row blocks: threads cost more than they save
        for h in range(nh):
            kh = h // inp["r"]
            O, H = head(inp["q"][:, kh], inp["k"][:, kh], inp["v"][:, h], inp["g"][:, h], inp["beta"][:, h],
                        inp["H0"][h], inp["scale"], cfg, scales)
            outs.append(O)
            Hs.append(H)
    o = np.stack(outs, 1)
    return gated_rmsnorm(o, inp["z"], inp["norm_w"], inp["rms_eps"]), np.stack(Hs)


def errors(ref, got):
    """(max |out error|, max over heads of max |H error| / max |H|)."""
    (o0, H0), (o1, H1) = ref, got
    eo = float(np.abs(o1 - o0).max())
    es = float((np.abs(H1 - H0).max(axis=(1, 2)) / np.abs(H0).max(axis=(1, 2))).max())
    return eo, es
