"""The layer's invariants checked through the GPU kernels (the oracle's own pins are in test_oracle_pins.py):

  * exact write: a token with g = 0 and beta = 1 leaves a state S with S k = v for its (unit) key k;
  * padding: a token with g = 0 and beta = 0 changes nothing, so an all-padding call leaves state and
    tail bit for bit as they were, and a call padded to a bucket ends in exactly the state (and emits
    exactly the outputs) of the call of the real length;
  * nothing is written outside the buffers: every output, state and checkpoint buffer carries canary
    margins that must come back untouched.

Run on an MI355X: python -u -m pytest tests -m gpu -x -v --timeout 300 --timeout-method thread
"""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_44_amd as gdn
from gdn_inputs import NEXT, LayerDims, make_inputs, make_layer, path_inputs, random_state
from tests.gpu_helpers import BOTH, Guarded, act, assert_state_close, desc_of, f32, host, i32, prefill_path, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    gdn.load_library()


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _write_token(x, t):
    """Make token t of every sequence an exact write: a = -inf (g = -exp(A_log) softplus(-inf) = 0) and
    b = +inf (beta = sigmoid(+inf) = 1); both are exact in bf16."""
    x.a[:, t] = -np.inf
    x.b[:, t] = np.inf


def _unit_keys_and_values(dims: LayerDims, w, mixed, tail0, t):
    """k^ (L2-normalised) and v of token t of one sequence, from the oracle's conv on the same inputs."""
    y, _ = oracle.conv(w.conv_w, tail0, mixed, mixed.shape[0])
    nk, dk = dims.n_k, dims.d_k
    k = y[t, nk * dk:2 * nk * dk].reshape(nk, dk)
    k = k / np.sqrt((k * k).sum(-1, keepdims=True) + dims.l2_eps)
    v = y[t, 2 * nk * dk:].reshape(dims.n_v, dims.d_v)
    return k, v


def _check_exact_write(dims: LayerDims, H, k, v, what):
    """S k = v with S = H^T for every value head (key head h // r), within 1e-3 of max|v| per head."""
    r = dims.n_v // dims.n_k
    for h in range(dims.n_v):
        got = H[h].T @ k[h // r]
        err = np.abs(got - v[h]).max() / max(np.abs(v[h]).max(), 1e-30)
        assert err <= 1e-3, f"{what}: head {h}: |S k - v| / max|v| = {err:.2e}"


@pytest.mark.parametrize("path", BOTH)
@pytest.mark.parametrize("L", [1, 64, 203])
def test_exact_write_prefill(path, L):
    """The last token of each sequence writes exactly (g = 0, beta = 1): the final state maps its key to
    its value, from a non-zero saved state, through both prefill paths."""
    dims = LayerDims(n_k=2, n_v=4, d_k=128, d_v=128)
    B = 2
    _say(f"exact write prefill path={path} L={L}")
    w, x, rng = make_layer(21, dims, B, L)
    _write_token(x, L - 1)
    H0, t0 = random_state(rng, dims, B)
    d = desc_of(dims)
    st, tail = f32(H0), act(t0, dims)
    with prefill_path(path):
        gdn.prefill_chunk(d, weights(w, dims), act(x.mixed, dims), act(x.z, dims), act(x.a, dims), act(x.b, dims),
                          i32(x.lens), tail, st)
    torch.cuda.synchronize()
    od = oracle.Dims.of(dims)
    for s in range(B):
        k, v = _unit_keys_and_values(dims, w, x.mixed[s], t0[s], L - 1)
        _check_exact_write(dims, host(st[s]), k, v, f"seq {s}")
        ref = oracle.layer_forward(od, w, x.mixed[s:s + 1], x.z[s:s + 1], x.a[s:s + 1], x.b[s:s + 1], None,
                                   t0[s:s + 1], H0[s:s + 1])
        assert_state_close(host(st[s]), ref["H"][0], f"state seq {s}")


def test_exact_write_decode():
    """A decode token with g = 0 and beta = 1 leaves S k = v."""
    dims, B = NEXT, 8
    _say("exact write decode")
    w, _, rng = make_layer(22, dims, 1, 1)
    H0, t0 = random_state(rng, dims, B)
    x = make_inputs(rng, dims, B, 1)
    _write_token(x, 0)
    d = desc_of(dims)
    sp, tp = f32(H0), act(t0, dims)
    gdn.decode_step(d, weights(w, dims), act(x.mixed[:, 0], dims), act(x.z[:, 0], dims), act(x.a[:, 0], dims),
                    act(x.b[:, 0], dims), None, tp, sp)
    torch.cuda.synchronize()
    for s in range(B):
        k, v = _unit_keys_and_values(dims, w, x.mixed[s], t0[s], 0)
        _check_exact_write(dims, host(sp[s]), k, v, f"decode seq {s}")


@pytest.mark.parametrize("path", BOTH)
@pytest.mark.parametrize("dims,B", [(LayerDims(n_k=2, n_v=4, d_k=128, d_v=128), 3), (NEXT, 8)])
def test_all_padding_call_leaves_state_bitwise(path, dims, B):
    """Every length 0: state and tail come back bit for bit, and no byte of the output is written."""
    L = 130
    _say(f"all padding path={path} B={B}")
    w, x, rng = make_layer(23, dims, B, L, [0] * B)
    H0, t0 = random_state(rng, dims, B)
    d = desc_of(dims)
    st = Guarded(dims.state_shape(B), torch.float32, f32(H0))
    tail = Guarded(dims.tail_shape(B), torch.bfloat16, act(t0, dims))
    out = Guarded((B, L, dims.value_dim), torch.bfloat16)
    out.t.view(torch.uint8).fill_(0xA5)  # the whole output as canary: nothing may be written
    with prefill_path(path):
        gdn.prefill_chunk(d, weights(w, dims), act(x.mixed, dims), act(x.z, dims), act(x.a, dims), act(x.b, dims),
                          i32(x.lens), tail.t, st.t, out.t)
    torch.cuda.synchronize()
    assert torch.equal(st.t, f32(H0)), "state changed"
    assert torch.equal(tail.t, act(t0, dims)), "tail changed"
    assert bool((out.raw == 0xA5).all()), "an all-padding call wrote output"
    st.check("state")
    tail.check("tail")


@pytest.mark.parametrize("path", BOTH)
@pytest.mark.parametrize("dims,B,n,bucket", [(LayerDims(n_k=2, n_v=4, d_k=128, d_v=128), 2, 100, 128),
                                             (LayerDims(n_k=2, n_v=4, d_k=128, d_v=128), 2, 1000, 1024),
                                             (NEXT, 8, 37, 64), (NEXT, 8, 300, 512)])
def test_bucket_padding_bitwise(path, dims, B, n, bucket):
    """A call whose chunk is padded to its bucket (padding rows random, masked by the length) ends in the
    same state and tail bits, and emits the same output bits on the real rows, as the call of exactly the
    real length."""
    _say(f"bucket padding path={path} B={B} n={n} bucket={bucket}")
    w, x, rng = make_layer(24, dims, B, bucket, [n] * B)
    H0, t0 = random_state(rng, dims, B)
    d = desc_of(dims)
    W = weights(w, dims)

    def run(L):
        st, tail = f32(H0), act(t0, dims)
        ins = [act(a[:, :L], dims) for a in (x.mixed, x.z, x.a, x.b)]
        with prefill_path(path):
            out = gdn.prefill_chunk(d, W, *ins, i32([n] * B), tail, st)
        torch.cuda.synchronize()
        return out[:, :n], st, tail

    o1, s1, t1 = run(n)
    o2, s2, t2 = run(bucket)
    assert torch.equal(s1, s2), "state bits differ between the exact and the bucket-padded call"
    assert torch.equal(t1, t2), "tail bits differ"
    assert torch.equal(o1, o2), "output bits differ on the real rows"


@pytest.mark.parametrize("dims", [LayerDims(n_k=2, n_v=4, d_k=64, d_v=128), LayerDims(n_k=2, n_v=6, d_k=128, d_v=32)])
def test_unequal_head_dims_padding_bitwise(dims):
    """Key and value heads of different dims (prefill on zero-padded copies): an all-padding call leaves
    state and tail bit for bit and writes no output byte; a bucket-padded call ends in the state, tail
    and real-row output bits of the call of exactly the real length."""
    B, n, bucket = 2, 100, 128
    _say(f"unequal head dims padding dims={dims}")
    w, x, rng = make_layer(25, dims, B, bucket, [n] * B)
    H0, t0 = random_state(rng, dims, B)
    d = desc_of(dims)
    W = weights(w, dims)
    st = Guarded(dims.state_shape(B), torch.float32, f32(H0))
    tail = Guarded(dims.tail_shape(B), torch.bfloat16, act(t0, dims))
    out = Guarded((B, bucket, dims.value_dim), torch.bfloat16)
    out.t.view(torch.uint8).fill_(0xA5)
    ins = [act(a, dims) for a in (x.mixed, x.z, x.a, x.b)]
    gdn.prefill_chunk(d, W, *ins, i32([0] * B), tail.t, st.t, out.t)
    torch.cuda.synchronize()
    assert torch.equal(st.t, f32(H0)), "state changed"
    assert torch.equal(tail.t, act(t0, dims)), "tail changed"
    assert bool((out.raw == 0xA5).all()), "an all-padding call wrote output"
    st.check("state")
    tail.check("tail")

    def run(L):
        s_, t_ = f32(H0), act(t0, dims)
        o_ = gdn.prefill_chunk(d, W, *[a[:, :L].contiguous() for a in ins], i32([n] * B), t_, s_)
        torch.cuda.synchronize()
        return o_[:, :n], s_, t_

    o1, s1, t1 = run(n)
    o2, s2, t2 = run(bucket)
    assert torch.equal(s1, s2) and torch.equal(t1, t2), "state or tail bits differ between exact and bucket call"
    assert torch.equal(o1, o2), "output bits differ on the real rows"


def test_canaries_decode_verify_paths():
    """Decode, verify and tree verify write nothing outside out, the pools and the checkpoint buffers."""
    dims, B, K, P = NEXT, 6, 4, 3
    T = K + 1
    _say("canaries decode / verify / paths")
    w, _, rng = make_layer(25, dims, 1, 1)
    H0, t0 = random_state(rng, dims, B)
    W = weights(w, dims)
    for out_f32 in (False, True):
        d = desc_of(dims, out_f32)
        x = make_inputs(rng, dims, B, T)
        sp = Guarded(dims.state_shape(B), torch.float32, f32(H0))
        tp = Guarded(dims.tail_shape(B), torch.bfloat16, act(t0, dims))
        out = Guarded((B, dims.value_dim), d.out)
        gdn.decode_step(d, W, act(x.mixed[:, 0], dims), act(x.z[:, 0], dims), act(x.a[:, 0], dims),
                        act(x.b[:, 0], dims), None, tp.t, sp.t, out.t)
        cks = Guarded((B, T, dims.n_v, dims.d_k, dims.d_v), torch.float32)
        ckt = Guarded((B, T, dims.kc, dims.conv_dim), torch.bfloat16)
        vout = Guarded((B, T, dims.value_dim), d.out)
        gdn.verify_with_checkpoints(d, W, act(x.mixed, dims), act(x.z, dims), act(x.a, dims), act(x.b, dims), None,
                                    tp.t, sp.t, cks.t, ckt.t, vout.t)
        xp = path_inputs(rng, dims, B, P, T)
        pcks = Guarded((B, P, T, dims.n_v, dims.d_k, dims.d_v), torch.float32)
        pckt = Guarded((B, P, T, dims.kc, dims.conv_dim), torch.bfloat16)
        pout = Guarded((B, P, T, dims.value_dim), d.out)
        gdn.verify_paths(d, W, act(xp.mixed, dims), act(xp.z, dims), act(xp.a, dims), act(xp.b, dims), None, tp.t,
                         sp.t, pcks.t, pckt.t, pout.t)
        torch.cuda.synchronize()
        for g, name in ((sp, "state pool"), (tp, "tail pool"), (out, "decode out"), (cks, "ckpt_state"),
                        (ckt, "ckpt_tail"), (vout, "verify out"), (pcks, "path ckpt_state"),
                        (pckt, "path ckpt_tail"), (pout, "paths out")):
            g.check(f"{name} (out_f32={out_f32})")


@pytest.mark.parametrize("path", BOTH)
def test_large_saved_state_range(path):
    """Saved states far above unit scale: std 30 (|S| up to ~140) stays inside the prefill's operand range
    and matches the oracle (fp32 outputs at 2e-3, state at 1e-3 of its max); std 400 leaves it, and the
    call reports that through the device status word instead of passing silently."""
    from tests.gpu_helpers import assert_out_flat
    dims = LayerDims(n_k=2, n_v=4, d_k=128, d_v=128)
    B, L = 2, 200
    w, x, rng = make_layer(26, dims, B, L)
    t0 = random_state(rng, dims, B)[1]
    od = oracle.Dims.of(dims)
    d = desc_of(dims, True)
    for std, in_range in ((30.0, True), (400.0, False)):
        _say(f"large saved state path={path} std={std}")
        H0 = (rng.standard_normal(dims.state_shape(B)) * std).astype(np.float32)
        gdn.device_status(clear=True)
        st, tail = f32(H0), act(t0, dims)
        with prefill_path(path):
            out = gdn.prefill_chunk(d, weights(w, dims), act(x.mixed, dims), act(x.z, dims), act(x.a, dims),
                                    act(x.b, dims), i32(x.lens), tail, st)
        status = gdn.device_status(clear=True)
        if in_range:
            assert status == 0, status
            for s in range(B):
                ref = oracle.layer_forward(od, w, x.mixed[s:s + 1], x.z[s:s + 1], x.a[s:s + 1], x.b[s:s + 1], None,
                                           t0[s:s + 1], H0[s:s + 1])
                assert_out_flat(host(out[s]), ref["out"][0], f"out seq {s}")
                assert_state_close(host(st[s]), ref["H"][0], f"state seq {s}")
        else:
            assert status & gdn.GDN_STATUS_RANGE, "a state beyond the operand range went unreported"


def test_two_runs_bitwise():
    """Every launch is deterministic: the same inputs give the same bits twice (prefill on both paths and
    on zero-padded heads, decode, verify with checkpoints, tree verify, accept and the state copy)."""
    dims, B, K, P = NEXT, 4, 4, 3
    T = K + 1
    _say("two runs bitwise")
    w, x, rng = make_layer(41, dims, 8, 300, [300, 1, 64, 250, 300, 200, 129, 300])
    H0, t0 = random_state(rng, dims, 8)
    W = weights(w, dims)
    d = desc_of(dims)
    ins = [act(a, dims) for a in (x.mixed, x.z, x.a, x.b)] + [i32(x.lens)]

    def prefill(path):
        st, tail = f32(H0), act(t0, dims)
        with prefill_path(path):
            out = gdn.prefill_chunk(d, W, *ins, tail, st)
        torch.cuda.synchronize()
        return out, st, tail

    for path in BOTH:
        a, b = prefill(path), prefill(path)
        for s, n in enumerate(x.lens):  # rows past a sequence's length are not outputs (left unwritten)
            assert torch.equal(a[0][s, :n], b[0][s, :n]), f"prefill ({path}) out of sequence {s} differs"
        for u, v, name in zip(a[1:], b[1:], ("state", "tail")):
            assert torch.equal(u, v), f"prefill ({path}) {name} differs between two runs"

    # prefill with key and value heads of different dims (zero-padded copies in the workspace)
    du = LayerDims(n_k=2, n_v=4, d_k=64, d_v=128)
    wu, xu, ru = make_layer(42, du, 2, 200, [200, 77])
    Hu, tu = random_state(ru, du, 2)
    Wu, dd = weights(wu, du), desc_of(du)
    insu = [act(a, du) for a in (xu.mixed, xu.z, xu.a, xu.b)] + [i32(xu.lens)]

    def prefill_unequal():
        st, tail = f32(Hu), act(tu, du)
        out = gdn.prefill_chunk(dd, Wu, *insu, tail, st)
        torch.cuda.synchronize()
        return out, st, tail

    a, b = prefill_unequal(), prefill_unequal()
    for s, n in enumerate(xu.lens):
        assert torch.equal(a[0][s, :n], b[0][s, :n]), f"unequal-dims prefill out of sequence {s} differs"
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2]), "unequal-dims prefill state or tail differs"

    xs = make_inputs(rng, dims, B, T)
    sp, tp = f32(H0[:B]), act(t0[:B], dims)
    step_in = [act(a, dims) for a in (xs.mixed, xs.z, xs.a, xs.b)]

    def decode():
        s2, t2 = sp.clone(), tp.clone()
        o = gdn.decode_step(d, W, *[a[:, 0].contiguous() for a in step_in], None, t2, s2)
        torch.cuda.synchronize()
        return o, s2, t2

    assert all(torch.equal(u, v) for u, v in zip(decode(), decode())), "decode differs between two runs"

    def verify():
        r = gdn.verify_with_checkpoints(d, W, *step_in, None, tp, sp)
        torch.cuda.synchronize()
        return r

    assert all(torch.equal(u, v) for u, v in zip(verify(), verify())), "verify differs between two runs"

    xp = path_inputs(rng, dims, B, P, T)
    path_in = [act(a, dims) for a in (xp.mixed, xp.z, xp.a, xp.b)]

    def paths():
        r = gdn.verify_paths(d, W, *path_in, None, tp, sp)
        torch.cuda.synchronize()
        return r

    assert all(torch.equal(u, v) for u, v in zip(paths(), paths())), "tree verify differs between two runs"

    drafts = i32(rng.integers(0, 3, size=(B, K)))
    preds = i32(rng.integers(0, 3, size=(B, K + 1)))
    a1, a2 = gdn.accept(drafts, preds), gdn.accept(drafts, preds)
    assert all(torch.equal(u, v) for u, v in zip(a1, a2)), "accept differs between two runs"
    ck_s, ck_t, _ = verify()

    def commit():
        s2, t2 = sp.clone(), tp.clone()
        gdn.state_copy(d, s2, t2, i32(np.arange(B)), ck_s, ck_t, a1[3], B)
        torch.cuda.synchronize()
        return s2, t2

    assert all(torch.equal(u, v) for u, v in zip(commit(), commit())), "state copy differs between two runs"


# ---- overlapping calls: two prefill calls on two streams, each with a workspace of its own -----------

_OVERLAP_SHAPES = {
    # (dims, B, L, lens): which kernels each takes is pinned in test_prefill_fused_launches and
    # test_prefill_norm_mode_launches
    "fused": (NEXT, 6, 300, [300, 1, 64, 250, 300, 200]),                                  # 192 units
    "two_phase": (LayerDims(n_k=16, n_v=16, d_k=128, d_v=128), 2, 300, [300, 129]),         # 32 units
    "exchange": (LayerDims(n_k=16, n_v=16, d_k=128, d_v=128), 3, 1030, [1030, 0, 700]),     # slices exchange row sums
}


@pytest.mark.parametrize("pair", [("fused", "fused"), ("two_phase", "two_phase"), ("exchange", "exchange"),
                                  ("fused", "exchange")])
def test_prefill_overlapping_calls_on_two_streams(pair):
    """Calls that may overlap need only workspaces of their own: two prefill calls issued back to back on
    two streams give, each, the bits of the same call run alone."""
    _say(f"overlapping prefill calls {pair}")
    calls = []
    for i, kind in enumerate(pair):
        dims, B, L, lens = _OVERLAP_SHAPES[kind]
        w, x, rng = make_layer(60 + i, dims, B, L, lens)
        H0, t0 = random_state(rng, dims, B)
        calls.append(dict(d=desc_of(dims), W=weights(w, dims), lens=lens, out_shape=(B, L, dims.value_dim),
                          ins=[act(a, dims) for a in (x.mixed, x.z, x.a, x.b)] + [i32(x.lens)],
                          H0=f32(H0), t0=act(t0, dims), ws_args=(B, L)))

    def buffers(c):
        return (c["H0"].clone(), c["t0"].clone(), torch.zeros(c["out_shape"], dtype=torch.bfloat16, device="cuda"),
                gdn.prefill_workspace(c["d"], *c["ws_args"]))

    def launch(c, buf):
        st, tail, out, ws = buf
        gdn.prefill_chunk(c["d"], c["W"], *c["ins"], tail, st, out, ws)

    alone = []
    for c in calls:
        buf = buffers(c)
        launch(c, buf)
        torch.cuda.synchronize()
        alone.append(buf)
    together = [buffers(c) for c in calls]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for c, buf, s in zip(calls, together, streams):
        with torch.cuda.stream(s):
            launch(c, buf)
    torch.cuda.synchronize()
    for k, (c, a, t) in enumerate(zip(calls, alone, together)):
        assert torch.equal(a[0], t[0]) and torch.equal(a[1], t[1]), f"call {k} ({pair[k]}): state or tail differs"
        for s, n in enumerate(c["lens"]):
            assert torch.equal(a[2][s, :n], t[2][s, :n]), f"call {k} ({pair[k]}): out of sequence {s} differs"


def test_step_batch_row_equals_batch_one():
    """A batch row equals batch = 1: decode and verify of 8 sequences give, for sequences 0, 3 and 7 run
    alone, the same output, state, checkpoint and tail bits (each sequence's steps do the same
    arithmetic whatever the batch)."""
    dims, B, T = NEXT, 8, 5
    _say("batch row = batch one (decode, verify)")
    w, _, rng = make_layer(43, dims, 1, 1)
    H0, t0 = random_state(rng, dims, B)
    x = make_inputs(rng, dims, B, T)
    d, W = desc_of(dims), weights(w, dims)
    ins = [act(a, dims) for a in (x.mixed, x.z, x.a, x.b)]
    sp, tp = f32(H0), act(t0, dims)
    out_b = gdn.decode_step(d, W, *[a[:, 0].contiguous() for a in ins], None, tp, sp)
    ck_s, ck_t, vout = gdn.verify_with_checkpoints(d, W, *ins, None, act(t0, dims), f32(H0))
    torch.cuda.synchronize()
    for s in (0, 3, 7):
        one = [a[s:s + 1].contiguous() for a in ins]
        sp1, tp1 = f32(H0[s:s + 1]), act(t0[s:s + 1], dims)
        o1 = gdn.decode_step(d, W, *[a[:, 0].contiguous() for a in one], None, tp1, sp1)
        c1s, c1t, v1 = gdn.verify_with_checkpoints(d, W, *one, None, act(t0[s:s + 1], dims), f32(H0[s:s + 1]))
        torch.cuda.synchronize()
        assert torch.equal(o1[0], out_b[s]) and torch.equal(sp1[0], sp[s]) and torch.equal(tp1[0], tp[s]), \
            f"decode of sequence {s} alone differs from its batch row"
        assert torch.equal(c1s[0], ck_s[s]) and torch.equal(c1t[0], ck_t[s]) and torch.equal(v1[0], vout[s]), \
            f"verify of sequence {s} alone differs from its batch row"
