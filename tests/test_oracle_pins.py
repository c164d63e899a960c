"""Pins of the fp64 oracle against what the layer's definition and mathematics fix (CPU only).

Each check is chosen so that a plausible slip in the oracle (a dropped term, a sign, an index, a
transposed state, a wrong head mapping or tail row) fails at least one of them. Shapes use
n_k != n_v and d_k != d_v so that transposes and head-mapping slips cannot cancel.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from gdn_inputs import LayerDims, LayerWeights, make_layer, chunk_lengths, ACT_F32
from tests import bruteforce as bf

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))


def _dims(n_k=2, n_v=4, d_k=8, d_v=12, scale=None, l2_eps=1e-6, rms_eps=1e-6):
    return oracle.Dims(n_k, n_v, d_k, d_v, 4, scale, l2_eps, rms_eps)


def _rand_core(rng, L, d, strong=False):
    q = rng.standard_normal((L, d.n_k, d.d_k))
    k = rng.standard_normal((L, d.n_k, d.d_k))
    v = rng.standard_normal((L, d.n_v, d.d_v))
    lo, hi = (0.0, np.log(16.0)) if strong else (np.log(0.05), np.log(0.5))
    A = np.exp(rng.uniform(lo, hi, d.n_v))
    g = -A * np.logaddexp(0.0, rng.standard_normal((L, d.n_v)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((L, d.n_v))))
    return q, k, v, g, beta


# ---- hand-worked fixtures -----------------------------------------------------------------------

def test_golden_two_token_delta_rule():
    c = GOLD["delta_rule_two_tokens"]
    dd = c["dims"]
    d = oracle.Dims(dd["n_k"], dd["n_v"], dd["d_k"], dd["d_v"], 4, dd["scale"], dd["l2_eps"], 1e-6)
    q, k, v = np.array(c["q"]), np.array(c["k"]), np.array(c["v"])
    g, beta = np.array(c["g"]), np.array(c["beta"])
    o0, H0 = oracle.delta_rule(d, q[:1], k[:1], v[:1], g[:1], beta[:1])
    np.testing.assert_allclose(H0, c["H_after_t0"], atol=1e-14)
    o, H = oracle.delta_rule(d, q, k, v, g, beta)
    np.testing.assert_allclose(o, c["o"], atol=1e-14)
    np.testing.assert_allclose(H, c["H_final"], atol=1e-14)


def test_golden_gates():
    c = GOLD["gates"]
    g, beta = oracle.gates(c["A_log"], c["dt_bias"], c["a"], c["b"], length=c["len"])
    np.testing.assert_allclose(g, c["g"], atol=1e-15)
    np.testing.assert_allclose(beta, c["beta"], atol=1e-15)


def test_golden_conv_and_tail():
    c = GOLD["conv"]
    pre = np.array(c["pre"])
    for n, key in ((2, "tail_len2"), (1, "tail_len1"), (0, "tail_len0")):
        y, tail = oracle.conv(c["w"], c["tail"], c["x"], length=n)
        np.testing.assert_allclose(y, pre / (1.0 + np.exp(-pre)), rtol=1e-15)
        np.testing.assert_array_equal(tail, c[key])


def test_golden_gated_rmsnorm():
    c = GOLD["gated_rmsnorm"]
    out = oracle.gated_rmsnorm(c["o"], c["z"], c["w"], 0.0)
    np.testing.assert_allclose(out, c["out"], atol=1e-14)


def test_golden_accept():
    c = GOLD["accept"]
    m, em, ne = oracle.accept(c["drafts"], c["preds"])
    np.testing.assert_array_equal(m, c["m"])
    np.testing.assert_array_equal(em, c["emitted"])
    np.testing.assert_array_equal(ne, c["n_emitted"])


def test_golden_accept_paths():
    c = GOLD["accept_paths"]
    m, path, em, ne = oracle.accept_paths(c["drafts"], c["preds"])
    np.testing.assert_array_equal(m, c["m"])
    np.testing.assert_array_equal(path, c["path"])
    np.testing.assert_array_equal(em, c["emitted"])
    np.testing.assert_array_equal(ne, c["n_emitted"])
    P, K = np.array(c["drafts"]).shape[1:]
    np.testing.assert_array_equal((np.arange(len(m)) * P + path) * (K + 1) + m, c["ckpt_index"])


# ---- P1: brute force (dense closed form, one triangular solve) ----------------------------------

@pytest.mark.parametrize("L,strong,h0", [(1, False, False), (7, False, True), (33, True, True), (64, False, True)])
def test_core_matches_dense_closed_form(L, strong, h0):
    rng = np.random.default_rng(100 + L)
    d = _dims()
    q, k, v, g, beta = _rand_core(rng, L, d, strong)
    H0 = rng.standard_normal((d.n_v, d.d_k, d.d_v)) if h0 else np.zeros((d.n_v, d.d_k, d.d_v))
    o, H = oracle.delta_rule(d, q, k, v, g, beta, H0)
    o_ref, H_ref = bf.delta_rule(q, k, v, g, beta, H0, d.d_k ** -0.5, d.l2_eps)
    np.testing.assert_allclose(o, o_ref, atol=1e-10, rtol=1e-10)
    np.testing.assert_allclose(H, H_ref, atol=1e-10, rtol=1e-10)


def test_scale_parameter():
    rng = np.random.default_rng(5)
    d1, d2 = _dims(scale=1.0), _dims(scale=0.25)
    q, k, v, g, beta = _rand_core(rng, 9, d1)
    o1, H1 = oracle.delta_rule(d1, q, k, v, g, beta)
    o2, H2 = oracle.delta_rule(d2, q, k, v, g, beta)
    np.testing.assert_array_equal(H1, H2)
    np.testing.assert_allclose(o2, 0.25 * o1, rtol=1e-14)


def test_gqa_head_mapping():
    """Value head h must read key head h // (n_v/n_k): compare against single-head runs."""
    rng = np.random.default_rng(6)
    d = _dims(n_k=2, n_v=6)
    q, k, v, g, beta = _rand_core(rng, 10, d)
    o, H = oracle.delta_rule(d, q, k, v, g, beta)
    d1 = _dims(n_k=1, n_v=1)
    for h in range(6):
        kh = h // 3
        o1, H1 = oracle.delta_rule(d1, q[:, kh:kh + 1], k[:, kh:kh + 1], v[:, h:h + 1], g[:, h:h + 1],
                                   beta[:, h:h + 1])
        np.testing.assert_array_equal(o[:, h], o1[:, 0])
        np.testing.assert_array_equal(H[h], H1[0])


# ---- P2: chunk form equals token by token --------------------------------------------------------

@pytest.mark.parametrize("C", [1, 5, 16, 64, 80])
def test_chunked_form_equals_tokenwise(C):
    rng = np.random.default_rng(7)
    d = _dims()
    L = 80
    q, k, v, g, beta = _rand_core(rng, L, d, strong=True)
    H0 = rng.standard_normal((d.n_v, d.d_k, d.d_v))
    o, H = oracle.delta_rule(d, q, k, v, g, beta, H0)
    o_c, H_c = bf.delta_rule(q, k, v, g, beta, H0, d.d_k ** -0.5, d.l2_eps, C=C)
    np.testing.assert_allclose(o_c, o, atol=1e-10, rtol=1e-10)
    np.testing.assert_allclose(H_c, H, atol=1e-10, rtol=1e-10)


# ---- P3: padding leaves the state unchanged ------------------------------------------------------

def test_padding_token_leaves_state_bit_identical():
    dims = LayerDims(n_k=2, n_v=4, d_k=8, d_v=12, act=ACT_F32)
    od = oracle.Dims.of(dims)
    w, x, rng = make_layer(11, dims, 1, 20)
    H0 = rng.standard_normal((1, 4, 8, 12))
    t0 = rng.standard_normal((1, 3, dims.conv_dim))
    r13 = oracle.layer_forward(od, w, x.mixed[:, :13], x.z[:, :13], x.a[:, :13], x.b[:, :13], None, t0, H0)
    rpad = oracle.layer_forward(od, w, x.mixed, x.z, x.a, x.b, [13], t0, H0)
    np.testing.assert_array_equal(rpad["H"], r13["H"])
    np.testing.assert_array_equal(rpad["tail"], r13["tail"])
    np.testing.assert_array_equal(rpad["out"][:, :13], r13["out"])
    # an all-padding call changes nothing
    r0 = oracle.layer_forward(od, w, x.mixed, x.z, x.a, x.b, [0], t0, H0)
    np.testing.assert_array_equal(r0["H"], H0)
    np.testing.assert_array_equal(r0["tail"], t0)


# ---- P4: exact write -----------------------------------------------------------------------------

def test_exact_write_retrieves_v():
    rng = np.random.default_rng(12)
    d = oracle.Dims(1, 1, 16, 10, 4, 1.0, 0.0, 1e-6)
    # orthonormal keys: every written value is retrieved exactly with g = 0, beta = 1
    Qm, _ = np.linalg.qr(rng.standard_normal((16, 16)))
    n = 9
    k = Qm[:, :n].T.reshape(n, 1, 16)
    v = rng.standard_normal((n, 1, 10))
    H0 = rng.standard_normal((1, 16, 10))
    g = np.zeros((n, 1))
    beta = np.ones((n, 1))
    o, H = oracle.delta_rule(d, k, k, v, g, beta, H0)
    for i in range(n):
        np.testing.assert_allclose(H[0].T @ k[i, 0], v[i, 0], atol=1e-12)  # S k_i = v_i
        np.testing.assert_allclose(o[i, 0], v[i, 0], atol=1e-12)            # o_t = S_t k_t = v_t
    # a direction orthogonal to all written keys still reads H0
    kperp = Qm[:, n]
    np.testing.assert_allclose(H[0].T @ kperp, H0[0].T @ kperp, atol=1e-12)


# ---- P5: beta = 0 closed form --------------------------------------------------------------------

def test_beta_zero_pure_decay():
    rng = np.random.default_rng(13)
    d = _dims()
    q, k, v, g, _ = _rand_core(rng, 12, d)
    beta = np.zeros_like(g)
    H0 = rng.standard_normal((d.n_v, d.d_k, d.d_v))
    o, H = oracle.delta_rule(d, q, k, v, g, beta, H0)
    gam = np.cumsum(g, 0)
    np.testing.assert_allclose(H, np.exp(gam[-1])[:, None, None] * H0, rtol=1e-12)
    qn = np.repeat(bf.l2n(q, d.l2_eps), 2, axis=1)
    for t in range(12):
        for h in range(d.n_v):
            exp_o = d.d_k ** -0.5 * np.exp(gam[t, h]) * (H0[h].T @ qn[t, h])
            np.testing.assert_allclose(o[t, h], exp_o, rtol=1e-12, atol=1e-14)


# ---- the whole layer: conv, gates, norms against numpy primitives --------------------------------

@pytest.mark.parametrize("seed,B,L,lens", [(0, 1, 64, [64]), (1, 2, 37, [37, 20]), (2, 3, 5, [5, 2, 0])])
def test_layer_matches_numpy_composition(seed, B, L, lens):
    dims = LayerDims(n_k=2, n_v=4, d_k=8, d_v=12, act=ACT_F32)
    od = oracle.Dims.of(dims)
    w, x, rng = make_layer(seed, dims, B, L, lens)
    H0 = rng.standard_normal((B, 4, 8, 12)) * 0.3
    t0 = rng.standard_normal((B, 3, dims.conv_dim))
    r = oracle.layer_forward(od, w, x.mixed, x.z, x.a, x.b, x.lens, t0, H0, want_o=True)
    out, tail, H, o = bf.layer(dims, w, x.mixed, x.z, x.a, x.b, x.lens, t0, H0)
    np.testing.assert_allclose(r["H"], H, atol=1e-10, rtol=1e-9)
    np.testing.assert_array_equal(r["tail"], tail)
    for s in range(B):
        n = lens[s]
        np.testing.assert_allclose(r["o"][s, :n], o[s, :n], atol=1e-10, rtol=1e-9)
        np.testing.assert_allclose(r["out"][s, :n], out[s, :n], atol=1e-9, rtol=1e-9)


def test_conv_matches_correlate_random():
    rng = np.random.default_rng(3)
    C, L = 7, 11
    w = rng.standard_normal((C, 4))
    tail = rng.standard_normal((3, C))
    x = rng.standard_normal((L, C))
    for n in (0, 1, 2, 3, 6, 11):
        y, t = oracle.conv(w, tail, x, n)
        y_ref, t_ref = bf.conv_silu(w, tail, x, n)
        np.testing.assert_allclose(y, y_ref, rtol=1e-13, atol=1e-15)
        np.testing.assert_array_equal(t, t_ref)


def test_gated_rmsnorm_library_and_invariance():
    rng = np.random.default_rng(4)
    o = rng.standard_normal((6, 16))
    z = rng.standard_normal((6, 16))
    w = 1.0 + 0.1 * rng.standard_normal(16)
    out = oracle.gated_rmsnorm(o, z, w, 1e-6)
    ref = (torch.nn.functional.rms_norm(torch.tensor(o), (16,), torch.tensor(w), eps=1e-6)
           * torch.nn.functional.silu(torch.tensor(z))).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    out7 = oracle.gated_rmsnorm(7.0 * o, z, w, 0.0)
    np.testing.assert_allclose(out7, oracle.gated_rmsnorm(o, z, w, 0.0), rtol=1e-13)


def test_gates_library():
    rng = np.random.default_rng(8)
    a = rng.standard_normal((9, 5))
    b = rng.standard_normal((9, 5))
    A_log = rng.uniform(0, np.log(16), 5)
    dt = rng.normal(0, 0.1, 5)
    g, beta = oracle.gates(A_log, dt, a, b, length=6)
    sp = torch.nn.functional.softplus(torch.tensor(a + dt), threshold=1e9).numpy()
    np.testing.assert_allclose(g[:6], -np.exp(A_log) * sp[:6], rtol=1e-13)
    np.testing.assert_allclose(beta[:6], torch.sigmoid(torch.tensor(b)).numpy()[:6], rtol=1e-14)
    assert np.all(g[6:] == 0) and np.all(beta[6:] == 0)


# ---- P6: snapshot -> restore -> replay; P7: split invariance ------------------------------------

def test_snapshot_restore_replay():
    dims = LayerDims(n_k=2, n_v=4, d_k=8, d_v=12, act=ACT_F32)
    od = oracle.Dims.of(dims)
    w, x, rng = make_layer(21, dims, 1, 30)
    sl = lambda a, i, j: a[:, i:j]
    full = oracle.layer_forward(od, w, x.mixed, x.z, x.a, x.b)
    # run 12 tokens, snapshot; run 8 "rejected" tokens of other inputs; restore; replay 18 real ones
    r1 = oracle.layer_forward(od, w, sl(x.mixed, 0, 12), sl(x.z, 0, 12), sl(x.a, 0, 12), sl(x.b, 0, 12))
    snap = (r1["tail"].copy(), r1["H"].copy())
    junk = rng.standard_normal((1, 8, dims.conv_dim))
    oracle.layer_forward(od, w, junk, sl(x.z, 0, 8), sl(x.a, 0, 8), sl(x.b, 0, 8), None, r1["tail"], r1["H"])
    r2 = oracle.layer_forward(od, w, sl(x.mixed, 12, 30), sl(x.z, 12, 30), sl(x.a, 12, 30), sl(x.b, 12, 30),
                              None, snap[0], snap[1])
    np.testing.assert_allclose(r2["H"], full["H"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r2["out"], full["out"][:, 12:], rtol=1e-10, atol=1e-11)
    np.testing.assert_array_equal(r2["tail"], full["tail"])


def test_split_with_padded_buckets_equals_single_pass():
    dims = LayerDims(n_k=2, n_v=4, d_k=8, d_v=12, act=ACT_F32)
    od = oracle.Dims.of(dims)
    w, x, rng = make_layer(22, dims, 1, 150)
    full = oracle.layer_forward(od, w, x.mixed, x.z, x.a, x.b)
    parts = chunk_lengths(rng, 150, buckets=(2, 4, 8, 16, 32, 64))
    tail, H, t0, outs = None, None, 0, []
    for n, bucket in parts:
        pad = lambda a: np.concatenate([a[:, t0:t0 + n], rng.standard_normal((1, bucket - n, a.shape[2]))], 1)
        r = oracle.layer_forward(od, w, pad(x.mixed), pad(x.z), pad(x.a), pad(x.b), [n], tail, H)
        tail, H = r["tail"], r["H"]
        outs.append(r["out"][:, :n])
        t0 += n
    np.testing.assert_allclose(H, full["H"], rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(tail, full["tail"])
    np.testing.assert_allclose(np.concatenate(outs, 1), full["out"], rtol=1e-9, atol=1e-10)


# ---- P10: accept, exhaustive; P11: verify = repeated decode --------------------------------------

def test_accept_exhaustive_k4_vocab3():
    K = 4
    drafts = np.array(list(itertools.product(range(3), repeat=K)), np.int32)
    preds = np.array(list(itertools.product(range(3), repeat=K + 1)), np.int32)
    D = np.repeat(drafts, len(preds), 0)
    P = np.tile(preds, (len(drafts), 1))
    m, em, ne = oracle.accept(D, P)
    eq = (P[:, :K] == D).astype(np.int64)
    m_ref = np.cumprod(eq, axis=1).sum(axis=1)
    np.testing.assert_array_equal(m, m_ref)
    np.testing.assert_array_equal(ne, m_ref + 1)
    for i in np.random.default_rng(0).choice(len(D), 500, replace=False):
        mm = m_ref[i]
        exp = list(D[i, :mm]) + [P[i, mm]] + [0] * (K - mm)
        np.testing.assert_array_equal(em[i], exp)


def test_accept_paths_exhaustive_p2_k2_vocab2():
    """Every pair of paths over a vocabulary of 2 with K = 2: the winner is the first maximum of the
    per-path match counts (numpy's argmax), and P = 1 is the single-path rule."""
    K, P = 2, 2
    dr1 = np.array(list(itertools.product(range(2), repeat=K)), np.int32)
    pr1 = np.array(list(itertools.product(range(2), repeat=K + 1)), np.int32)
    one = [(d, q) for d in dr1 for q in pr1]                     # every (drafts, preds) of one path
    pairs = list(itertools.product(range(len(one)), repeat=P))   # every assignment of two paths
    D = np.array([[one[i][0] for i in pr] for pr in pairs])
    Q = np.array([[one[i][1] for i in pr] for pr in pairs])
    m, path, em, ne = oracle.accept_paths(D, Q)
    mp = np.cumprod(Q[:, :, :K] == D, axis=2).sum(axis=2)       # [cases, P]
    np.testing.assert_array_equal(m, mp.max(axis=1))
    np.testing.assert_array_equal(path, np.argmax(mp, axis=1))
    win = np.arange(len(pairs))
    m1, em1, ne1 = oracle.accept(D[win, path], Q[win, path])
    np.testing.assert_array_equal(em, em1)
    np.testing.assert_array_equal(ne, ne1)
    # one path: the same as accept
    m2, path2, em2, ne2 = oracle.accept_paths(D[:, :1], Q[:, :1])
    m3, em3, ne3 = oracle.accept(D[:, 0], Q[:, 0])
    assert not path2.any()
    np.testing.assert_array_equal(m2, m3)
    np.testing.assert_array_equal(em2, em3)


def test_verify_paths_rows_start_from_their_sequence():
    """Path p of sequence b is an ordinary verify from sequence b's state and tail; paths with the same
    tokens give the same checkpoints."""
    dims = LayerDims(n_k=1, n_v=2, d_k=4, d_v=6, act=ACT_F32)
    od = oracle.Dims.of(dims)
    B, P, T = 2, 3, 4
    w, x, rng = make_layer(29, dims, B * P, T)
    shape = lambda a: a.reshape((B, P) + a.shape[1:])
    mixed, z, a, b = shape(x.mixed).copy(), shape(x.z), shape(x.a), shape(x.b)
    mixed[1, 2] = mixed[1, 0]  # sequence 1: path 2 repeats path 0's tokens
    z, a, b = z.copy(), a.copy(), b.copy()
    z[1, 2], a[1, 2], b[1, 2] = z[1, 0], a[1, 0], b[1, 0]
    H0 = rng.standard_normal((B, 2, 4, 6)) * 0.3
    t0 = rng.standard_normal((B, 3, dims.conv_dim))
    r = oracle.verify_paths(od, w, mixed, z, a, b, t0, H0)
    for s in range(B):
        for p in range(P):
            one = oracle.verify(od, w, mixed[s, p:p + 1], z[s, p:p + 1], a[s, p:p + 1], b[s, p:p + 1], t0[s:s + 1],
                                H0[s:s + 1])
            for k in ("ckpt_H", "ckpt_tail", "out"):
                np.testing.assert_array_equal(r[k][s, p], one[k][0])
    for k in ("ckpt_H", "ckpt_tail", "out"):
        np.testing.assert_array_equal(r[k][1, 2], r[k][1, 0])
        assert not np.array_equal(r[k][0, 1], r[k][0, 0])


def test_verify_checkpoints_equal_repeated_decode():
    dims = LayerDims(n_k=2, n_v=4, d_k=8, d_v=12, act=ACT_F32)
    od = oracle.Dims.of(dims)
    w, x, rng = make_layer(23, dims, 3, 5)
    H0 = rng.standard_normal((3, 4, 8, 12)) * 0.2
    t0 = rng.standard_normal((3, 3, dims.conv_dim))
    ver = oracle.verify(od, w, x.mixed, x.z, x.a, x.b, t0, H0)
    tail, H = t0.copy(), H0.copy()
    for i in range(5):
        sl = lambda a: a[:, i:i + 1]
        r = oracle.layer_forward(od, w, sl(x.mixed), sl(x.z), sl(x.a), sl(x.b), None, tail, H)
        tail, H = r["tail"], r["H"]
        np.testing.assert_array_equal(ver["ckpt_H"][:, i], H)
        np.testing.assert_array_equal(ver["ckpt_tail"][:, i], tail)
        np.testing.assert_array_equal(ver["out"][:, i], r["out"][:, 0])
    # and the whole T-token run equals one multi-token call
    full = oracle.layer_forward(od, w, x.mixed, x.z, x.a, x.b, None, t0, H0)
    np.testing.assert_allclose(ver["ckpt_H"][:, -1], full["H"], rtol=1e-12, atol=1e-13)


# ---- the prefix-state cache's bookkeeping (qev_fast/statecache.py page), worked by hand ----------

def test_prefix_model_bounds_hand_worked():
    from oracle.prefix_cache import PrefixCacheModel
    m = PrefixCacheModel(8, stride=2048, tail=16, align=64)
    # stride multiples below p = 4992, p - tail = 4984 rounded down to 4928, and p
    assert m.chunk_ends(0, 5000) == [2048, 4096, 4928, 4992]
    assert m.chunk_ends(4096, 5000) == [4928, 4992]
    # p - tail rounds down to 0, not past the start: only p
    assert m.chunk_ends(0, 64) == [64]
    # no stride, no tail: p alone, cut into chunks of at most 2048
    assert PrefixCacheModel(8, stride=0, tail=0, max_chunk=2048).chunk_ends(0, 5000) == [2048, 4096, 4992]


def test_prefix_model_lookup_and_lru_hand_worked():
    from oracle.prefix_cache import PrefixCacheModel
    m = PrefixCacheModel(2, stride=2048, tail=16, align=64, min_prefix=256)
    A = np.arange(1000)
    B = np.concatenate([A[:500], -np.arange(1, 501)])
    D = np.arange(5000, 6000)
    # A: cold, one checkpoint at p = 960 (p - tail = 984 also rounds down to 960)
    assert m.row(A, 1000) == (-1, 0, 960, [960], [0])
    # B shares 500 tokens with A: checkpoint 0 (at 960) is past that, so cold again
    assert m.row(B, 1000) == (-1, 0, 960, [960], [1])
    # A again: a hit on checkpoint 0, which becomes the most recently used
    assert m.row(A, 1000) == (0, 960, 960, [], [])
    # D: cold; three checkpoints for two slots, so B's (the least recently used) goes
    assert m.row(D, 1000) == (-1, 0, 960, [960], [2])
    assert m.alive() == [0, 2]
    # B once more: its checkpoint is gone
    assert m.row(B, 1000)[:2] == (-1, 0)
    # a row below min_prefix takes the plain path
    assert m.row(A[:200], 200) == (-1, 0, 192, [], [])
    assert m.stats == dict(rows=5, hits=1, partial=0, cold=4, plain=1, tokens_reused=960,
                           tokens_computed=4 * 1000 + 40 + 200, ckpts_made=4, evicted=2, rows_kept=2)
    # the rows whose checkpoints are all gone are forgotten: A (checkpoint 0) and D (checkpoint 2) stay
    assert m.rows_remembered() == 2


def test_prefix_model_forgets_evicted_rows():
    """Many distinct rows through a small pool: the model keeps at most one row per live checkpoint."""
    from oracle.prefix_cache import PrefixCacheModel
    m = PrefixCacheModel(3, stride=512, tail=0, align=64, min_prefix=64)
    rng = np.random.default_rng(5)
    for _ in range(200):
        m.row(rng.integers(0, 1000, size=int(rng.integers(64, 1500))), 1500)
        assert m.rows_remembered() <= len(m.alive()) <= 3


# ---- the state record copy (uni_engine.py page, copy_cache_) -------------------------------------

def test_state_copy_hand_worked():
    """Rows of constant value: records 2 and 0 of the source go to rows 3 and 1 of the destination, only
    the first n = 2 index pairs count, and the other rows keep their values."""
    src = np.array([10.0, 11.0, 12.0, 13.0])[:, None] * np.ones((4, 3))
    tail = np.array([20, 21, 22, 23], np.uint16)[:, None] * np.ones((4, 2), np.uint16)
    dst, dtail = -np.ones((5, 3)), np.zeros((5, 2), np.uint16)
    oracle.state_copy(dst, dtail, [3, 1, 0], src, tail, [2, 0, 1], 2)
    np.testing.assert_array_equal(dst[:, 0], [-1.0, 10.0, -1.0, 12.0, -1.0])
    np.testing.assert_array_equal(dtail[:, 0], [0, 20, 0, 22, 0])


def test_state_copy_is_bitwise_and_round_trips():
    """NaN payloads and -0.0 survive as bits; a permutation and then its inverse give the source back;
    None indices copy rows 0..n-1; a repeated destination row is rejected."""
    rng = np.random.default_rng(3)
    src = rng.standard_normal((6, 4, 4)).astype(np.float32)
    src[1, 0, 0] = -0.0
    src[2].view(np.uint32)[0, 0] = 0x7FC01234  # a NaN with a payload
    perm = rng.permutation(6)
    mid = np.zeros_like(src)
    oracle.state_copy(mid, None, perm, src, None, None, 6)
    back = np.zeros_like(src)
    oracle.state_copy(back, None, None, mid, None, perm, 6)
    assert back.tobytes() == src.tobytes()
    ident = np.zeros_like(src)
    oracle.state_copy(ident, None, None, src, None, None, 4)
    assert ident[:4].tobytes() == src[:4].tobytes() and not ident[4:].any()
    with pytest.raises(ValueError):
        oracle.state_copy(np.zeros_like(src), None, [1, 1], src, None, [0, 2], 2)
