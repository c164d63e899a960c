"""GPU parity: every libgdn entry point against the fp64 oracle on the same seeded inputs.

Run on an MI355X: python -u -m pytest tests -m gpu -x -v --timeout 300 --timeout-method thread
"""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_44_amd as gdn
from gdn_inputs import (ACT_BF16, ACT_F32, NEXT, SMALL, TINY, LayerDims, chunk_lengths, make_layer, path_inputs,
                        random_state, verify_draws, verify_path_draws)
from tests.gpu_helpers import (BOTH, Guarded, act, assert_out_close, assert_out_flat, assert_state_close, desc_of, f32,
                               host, i32, out_excess, prefill_path, state_rel_err, weights)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    gdn.load_library()


def _say(msg):
    print(f"[case] {msg}", flush=True)


# ---------------------------------------------------------------------------------------------------
# prefill

def _prefill_case(dims: LayerDims, seed, B, L, lens, state_std=0.0, tail_rand=False, sample=None, paths=(None,)):
    """Inputs and the oracle once; then every requested path, with the output in the activation dtype and
    (bf16 activations) in fp32. Buffers carry canary margins; the fp32-output call must leave the same
    state and tail bits as the other."""
    _say(f"prefill seed={seed} B={B} L={L} lens={list(lens)[:4]} dims={dims} paths={paths}")
    w, x, rng = make_layer(seed, dims, B, L, lens)
    H0 = (rng.standard_normal(dims.state_shape(B)) * state_std).astype(np.float32)
    t0 = random_state(rng, dims, B)[1] if tail_rand else np.zeros(dims.tail_shape(B), np.float32)
    idx = range(B) if sample is None else sample
    od = oracle.Dims.of(dims)
    refs = {s: oracle.layer_forward(od, w, x.mixed[s:s + 1], x.z[s:s + 1], x.a[s:s + 1], x.b[s:s + 1],
                                    x.lens[s:s + 1], t0[s:s + 1], H0[s:s + 1]) for s in idx}
    inputs = [act(x.mixed, dims), act(x.z, dims), act(x.a, dims), act(x.b, dims), i32(x.lens)]
    W = weights(w, dims)
    result = None
    for path in paths:
        bits = None
        for out_f32 in ((False, True) if dims.act == ACT_BF16 else (False,)):
            d = desc_of(dims, out_f32)
            _say(f"  path={path} out_f32={out_f32}")
            tail = Guarded(dims.tail_shape(B), d.act, act(t0, dims))
            st = Guarded(dims.state_shape(B), torch.float32, f32(H0))
            out = Guarded((B, L, dims.value_dim), d.out)
            with prefill_path(path):
                gdn.prefill_chunk(d, W, *inputs, tail.t, st.t, out.t)
            torch.cuda.synchronize()
            for g, name in ((tail, "tail"), (st, "state"), (out, "out")):
                g.check(f"{name} (path {path})")
            for s in idx:
                n = int(x.lens[s])
                ref = refs[s]
                if out_f32:
                    assert_out_flat(host(out.t[s, :n]), ref["out"][0, :n], f"fp32 out[seq {s}] (path {path})")
                else:
                    assert_out_close(host(out.t[s, :n]), ref["out"][0, :n], dims, f"out[seq {s}] (path {path})")
                assert_state_close(host(st.t[s]), ref["H"][0], f"state[seq {s}] (path {path})")
                np.testing.assert_array_equal(host(tail.t[s]), ref["tail"][0].astype(np.float32))
            if bits is None:
                bits = (st.t.clone(), tail.t.clone())
            else:  # the output's dtype changes nothing else
                assert torch.equal(st.t, bits[0]) and torch.equal(tail.t, bits[1]), f"state bits differ (path {path})"
            if not out_f32:
                result = (out.t, st.t, tail.t)
    return result


def test_prefill_tiny_fp32():
    """The tiny CPU-checkable layer: T=64, 2 key / 4 value heads, d=32, fp32 I/O."""
    _prefill_case(TINY, 0, 1, 64, [64])


@pytest.mark.parametrize("D,R", [(32, 2), (64, 1), (128, 2), (128, 4)])
def test_prefill_ragged_multichunk(D, R):
    """Several chunks with a ragged tail and a padded sequence, from a non-zero state and tail."""
    dims = LayerDims(n_k=2, n_v=2 * R, d_k=D, d_v=D)
    _prefill_case(dims, 3, 3, 300, [300, 171, 1], state_std=0.05, tail_rand=True, paths=BOTH if D == 128 else (None,))


@pytest.mark.parametrize("B", [2, 4, 5, 8])
def test_prefill_column_splits_d128(B):
    """32 value heads x B sequences: 64, 128, 160 and 256 (sequence, head) pairs give 4, 2, 1 and 1
    state-pass workgroups per head; the split heads exchange their partial row sums for the gated norm."""
    lens = [150, 64, 1, 100, 129, 0, 150, 37][:B]
    _prefill_case(NEXT, 11, B, 150, lens, state_std=0.05, tail_rand=True, paths=BOTH)


@pytest.mark.parametrize("dims,B,L,lens", [(LayerDims(n_k=16, n_v=16, d_k=128, d_v=128), 3, 1030, [1030, 0, 700]),
                                            (LayerDims(n_k=24, n_v=24, d_k=128, d_v=128), 3, 1030, [1030, 1, 900]),
                                            (NEXT, 2, 1030, [1030, 999]),
                                            (NEXT, 3, 1030, [1030, 500, 1])])
def test_prefill_split_row_sum_exchange(dims, B, L, lens):
    """Calls of at least 1024 tokens with 32- or 64-column state-pass slices: the slices of a head
    exchange their partial row sums for the gated norm. 48 and 72 (sequence, head) pairs with one value
    head per key head, 64 and 96 with two; ragged lengths (one sequence empty), from a non-zero state
    and tail."""
    _prefill_case(dims, 12, B, L, lens, state_std=0.05, tail_rand=True, paths=BOTH)


@pytest.mark.parametrize("D,R,act_t", [(32, 1, ACT_BF16), (32, 4, ACT_BF16), (64, 4, ACT_BF16),
                                       (32, 1, ACT_F32), (32, 4, ACT_F32), (64, 1, ACT_F32),
                                       (64, 4, ACT_F32), (64, 3, ACT_BF16), (32, 6, ACT_F32),
                                       (128, 8, ACT_BF16), (128, 3, ACT_BF16), (128, 1, ACT_F32),
                                       (128, 2, ACT_F32), (128, 4, ACT_F32)])
def test_prefill_every_head_shape(D, R, act_t):
    """The remaining compiled (d, value heads per key head, activation type) combinations: ragged
    multi-chunk sequences from a non-zero state and tail. At d = 64 with four value heads per key head
    on fp32 activations, this seed makes one 2^8 beta v product land one fp32 ulp above an f16 tie: it
    fails by one f16 ulp of a U' element (2.3e-3 at the output) when a hi/lo split's two halves are
    rounded from different values."""
    dims = LayerDims(n_k=2, n_v=2 * R, d_k=D, d_v=D, act=act_t)
    paths = BOTH if D == 128 and act_t == ACT_BF16 else (None,)
    _prefill_case(dims, 8, 2, 150, [150, 67], state_std=0.05, tail_rand=True, paths=paths)


@pytest.mark.parametrize("dk,dv,R,act_t", [(64, 128, 2, ACT_BF16), (128, 64, 1, ACT_BF16), (128, 32, 4, ACT_BF16),
                                           (32, 64, 3, ACT_BF16), (32, 128, 2, ACT_F32), (64, 32, 1, ACT_F32)])
def test_prefill_unequal_head_dims(dk, dv, R, act_t):
    """Key and value heads of different dims (the square kernels at max(d_k, d_v) on zero-padded copies):
    ragged multi-chunk sequences from a non-zero state and tail, outputs in the activation dtype and in
    fp32, state and tail against the oracle, canaries around every output."""
    dims = LayerDims(n_k=2, n_v=2 * R, d_k=dk, d_v=dv, act=act_t)
    _prefill_case(dims, 21, 2, 150, [150, 67], state_std=0.05, tail_rand=True)


def _random_shape(seed):
    """A seeded layer shape and call: head dims from {32, 64, 128} (equal or drawn apart), GQA ratio
    1-4, one or two key heads, bf16 or fp32 activations, 1-3 sequences of ragged lengths (some empty)."""
    r = np.random.default_rng(1000 + seed)
    n_k, d_k = int(r.integers(1, 3)), int(r.choice([32, 64, 128]))
    d_v = d_k if r.random() < 0.4 else int(r.choice([32, 64, 128]))
    dims = LayerDims(n_k=n_k, n_v=n_k * int(r.integers(1, 5)), d_k=d_k, d_v=d_v,
                     act=ACT_F32 if r.random() < 0.3 else ACT_BF16)
    B = int(r.integers(1, 4))
    L = int(r.integers(1, 300))
    lens = [int(v) for v in r.integers(0, L + 1, size=B)]
    lens[int(r.integers(0, B))] = L
    return dims, B, L, lens


@pytest.mark.parametrize("seed", range(40))
def test_prefill_random_shapes(seed):
    """Seeded random shapes and ragged calls through prefill (both paths where the fused one is built),
    from a non-zero state and tail, against the oracle."""
    dims, B, L, lens = _random_shape(seed)
    paths = BOTH if dims.d_k == dims.d_v == 128 and dims.act == ACT_BF16 else (None,)
    _prefill_case(dims, 50 + seed, B, L, lens, state_std=0.05, tail_rand=True, paths=paths)


def _random_long_shape(seed):
    """A seeded longer call: 1-16 key heads, GQA ratio 1-4, head dims from {32, 64, 128}, bf16 or fp32,
    1-6 sequences of 300-4096 tokens (ragged, some empty), bounded so the oracle stays in seconds."""
    r = np.random.default_rng(5000 + seed)
    n_k, d_k = int(r.choice([1, 2, 4, 8, 16])), int(r.choice([32, 64, 128]))
    d_v = d_k if r.random() < 0.6 else int(r.choice([32, 64, 128]))
    dims = LayerDims(n_k=n_k, n_v=n_k * int(r.integers(1, 5)), d_k=d_k, d_v=d_v,
                     act=ACT_F32 if r.random() < 0.2 else ACT_BF16)
    B, L = int(r.integers(1, 7)), int(r.integers(300, 4097))
    lens = [int(v) for v in r.integers(0, L + 1, size=B)]
    lens[int(r.integers(0, B))] = L
    return dims, B, L, lens


@pytest.mark.parametrize("seed", range(14))
def test_prefill_random_long_shapes(seed):
    """Seeded longer calls (many chunks, column splits, row-sum exchanges, the fused path at its own unit
    counts) through prefill on both paths where the fused one is built, against the oracle."""
    dims, B, L, lens = _random_long_shape(seed)
    if sum(lens) * dims.n_v * dims.d_k * dims.d_v > 4e9:
        pytest.skip("beyond the oracle's time bound")
    paths = BOTH if dims.d_k == dims.d_v == 128 and dims.act == ACT_BF16 else (None,)
    _prefill_case(dims, 7000 + seed, B, L, lens, state_std=0.05, tail_rand=True, paths=paths)


@pytest.mark.parametrize("seed", range(24))
def test_decode_random_shapes(seed):
    """The same random shapes through decode, from saved states, against the oracle."""
    dims, B, _, _ = _random_shape(seed)
    _say(f"decode random seed={seed} B={B} dims={dims}")
    w, _, rng = make_layer(60 + seed, dims, 1, 1)
    H0, T0 = _saved_states(dims, w, rng, B)
    x = _decode_inputs(dims, rng, B, 1)
    d = desc_of(dims, True)
    sp, tp = f32(H0), act(T0, dims)
    out = gdn.decode_step(d, weights(w, dims), act(x.mixed[:, 0], dims), act(x.z[:, 0], dims),
                          act(x.a[:, 0], dims), act(x.b[:, 0], dims), None, tp, sp)
    torch.cuda.synchronize()
    ref = oracle.layer_forward(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, None, T0, H0)
    assert_out_flat(host(out), ref["out"][:, 0], "decode fp32 out")
    assert_state_close(host(sp), ref["H"])
    np.testing.assert_array_equal(host(tp), ref["tail"].astype(np.float32))


@pytest.mark.parametrize("seed", range(24))
def test_verify_paths_random_shapes(seed):
    """The random shapes through tree verify: 1-3 paths of 1+K tokens (K from 1 to 4) per sequence from
    permuted pool rows, fp32 outputs at the flat bound and every checkpoint against the oracle, the pool
    untouched, and the paths' shared first token leaving every path in the same bits."""
    dims, B, _, _ = _random_shape(seed)
    r = np.random.default_rng(2000 + seed)
    P, K = int(r.integers(1, 4)), int(r.integers(1, 5))
    T = K + 1
    _say(f"verify paths random seed={seed} B={B} P={P} K={K} dims={dims}")
    w, _, rng = make_layer(70 + seed, dims, 1, 1)
    H0, T0 = _saved_states(dims, w, rng, B)
    x = path_inputs(rng, dims, B, P, T)
    d = desc_of(dims, True)
    npool = B + 2
    slots = rng.permutation(npool)[:B].astype(np.int32)
    poolH = np.zeros(dims.state_shape(npool), np.float32)
    poolT = np.zeros(dims.tail_shape(npool), np.float32)
    poolH[slots], poolT[slots] = H0, T0
    sp, tp = f32(poolH), act(poolT, dims)
    ck_s, ck_t, out = gdn.verify_paths(d, weights(w, dims), act(x.mixed, dims), act(x.z, dims), act(x.a, dims),
                                       act(x.b, dims), i32(slots), tp, sp, check_slots=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(sp), poolH), "verify modified the pool"
    ref = oracle.verify_paths(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, T0, H0)
    assert_out_flat(host(out), ref["out"], "verify_paths fp32 out")
    cks = host(ck_s)
    for p in range(P):
        for i in range(T):
            assert_state_close(cks[:, p, i], ref["ckpt_H"][:, p, i], f"path {p} checkpoint {i}")
    np.testing.assert_array_equal(host(ck_t), ref["ckpt_tail"].astype(np.float32))
    for p in range(1, P):
        assert torch.equal(ck_s[:, p, 0], ck_s[:, 0, 0]) and torch.equal(out[:, p, 0], out[:, 0, 0])


def test_prefill_fp32_multichunk():
    dims = LayerDims(n_k=2, n_v=4, d_k=64, d_v=64, act=ACT_F32)
    _prefill_case(dims, 4, 2, 200, [200, 129], state_std=0.05, tail_rand=True)


def test_prefill_zero_length_leaves_state():
    dims = LayerDims(n_k=2, n_v=4, d_k=128, d_v=128)
    _prefill_case(dims, 5, 2, 64, [0, 2], state_std=0.05, tail_rand=True, paths=BOTH)


def test_prefill_4k_single_layer():
    """One sequence of 4096 tokens, 16 key / 16 value heads, d=128, bf16 activations, fp32 state."""
    _prefill_case(SMALL, 0, 1, 4096, [4096], paths=BOTH)


def test_prefill_streamed_records_ragged():
    """Two ragged sequences (4096 and 3000 tokens) at 16/32 heads: about 400 MB of chunk records, which
    the record builder stores non-temporally, and 64 (sequence, head) pairs, whose 32-column state-pass
    slices exchange row sums for the gated norm. Both sequences against the oracle."""
    _prefill_case(NEXT, 13, 2, 4096, [4096, 3000], state_std=0.05, tail_rand=True, paths=BOTH)


def test_prefill_stack_layer_sampled():
    """Stack-layer shape (8 x 8192 tokens, 16/32 heads) on the GPU; sequences 0 and 7 against the oracle."""
    _prefill_case(NEXT, 1, 8, 8192, [8192] * 8, sample=[0, 7], paths=BOTH)


def test_prefill_scale_one():
    dims = LayerDims(n_k=2, n_v=4, d_k=64, d_v=64, scale=1.0)
    _prefill_case(dims, 6, 1, 130, [130], state_std=0.05)


@pytest.mark.parametrize("path", BOTH)
def test_prefill_strong_decays(path):
    """Gates at the strong end inside chunks of ordinary tokens, from a saved state: runs of tokens with
    a = 40 or 12 (log-decays of -640 and -192 per token at A = 16) and single full forgets (a = +inf,
    g = -inf). The in-chunk sums of g then reach 10^4 in magnitude while the decays between the
    ordinary tokens after them stay near 1; both paths must still match the oracle."""
    dims = LayerDims(n_k=2, n_v=4, d_k=128, d_v=128)
    B, L, lens = 2, 300, [300, 171]
    _say(f"strong decays path={path}")
    w, x, rng = make_layer(31, dims, B, L, lens)
    w.A_log[:] = np.float32(np.log(16.0))
    w.A_log[0] = 0.0  # one slow head beside three fast ones
    x.a[:, 70:80] = 40.0
    x.a[:, 130] = np.inf
    x.a[0, 200:240] = 12.0
    x.a[0, 290] = np.inf
    H0, t0 = random_state(rng, dims, B)
    od = oracle.Dims.of(dims)
    d = desc_of(dims, out_f32=True)
    st, tail = f32(H0), act(t0, dims)
    out = torch.zeros(B, L, dims.value_dim, dtype=torch.float32, device="cuda")
    with prefill_path(path):
        gdn.prefill_chunk(d, weights(w, dims), act(x.mixed, dims), act(x.z, dims), act(x.a, dims), act(x.b, dims),
                          i32(x.lens), tail, st, out)
    torch.cuda.synchronize()
    for s in range(B):
        n = lens[s]
        ref = oracle.layer_forward(od, w, x.mixed[s:s + 1], x.z[s:s + 1], x.a[s:s + 1], x.b[s:s + 1],
                                   x.lens[s:s + 1], t0[s:s + 1], H0[s:s + 1])
        assert_out_flat(host(out[s, :n]), ref["out"][0, :n], f"fp32 out[seq {s}] (path {path})")
        assert_state_close(host(st[s]), ref["H"][0], f"state[seq {s}] (path {path})")
        np.testing.assert_array_equal(host(tail[s]), ref["tail"][0].astype(np.float32))


@pytest.mark.parametrize("dims", [LayerDims(n_k=2, n_v=4, d_k=128, d_v=128), LayerDims(n_k=2, n_v=6, d_k=64, d_v=64, act=ACT_F32),
                                  LayerDims(n_k=1, n_v=2, d_k=32, d_v=128)])
@pytest.mark.parametrize("parts", [[0, 0, 1, 1, 1], [0, 144, 22, 16, 8], [42, 129, 1], [2, 81, 89, 119]])
def test_continuation_tiny_calls(dims, parts):
    """One sequence cut into calls of 0, 1 or 2 real tokens among longer ones (a call of 0 still passes one
    padded row), each continuing from the last: the outputs, the final state and the conv tail match the
    oracle's single pass (calls shorter than the conv tail keep its older rows)."""
    total = sum(parts)
    _say(f"continuation tiny calls parts={parts} dims={dims}")
    w, x, rng = make_layer(90, dims, 1, total)
    H0, t0 = random_state(rng, dims, 1)
    ref = oracle.layer_forward(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, None, t0, H0)
    d, W = desc_of(dims, out_f32=True), weights(w, dims)
    for path in (BOTH if dims.d_k == dims.d_v == 128 and dims.act == ACT_BF16 else (None,)):
        st, tail = f32(H0), act(t0, dims)
        outs, pos = [], 0
        for n in parts:
            Lb = max(n, 1)
            seg = [np.concatenate([a[:, pos:pos + n], np.zeros((1, Lb - n, a.shape[2]), np.float32)], 1)
                   for a in (x.mixed, x.z, x.a, x.b)]
            out = torch.zeros(1, Lb, dims.value_dim, dtype=torch.float32, device="cuda")
            with prefill_path(path):
                gdn.prefill_chunk(d, W, *[act(a, dims) for a in seg], i32([n]), tail, st, out)
            torch.cuda.synchronize()
            outs.append(host(out[0, :n]))
            pos += n
        assert_out_flat(np.concatenate(outs, 0), ref["out"][0], f"continued out (path {path})")
        assert_state_close(host(st[0]), ref["H"][0], f"continued state (path {path})")
        np.testing.assert_array_equal(host(tail[0]), ref["tail"][0].astype(np.float32))


def test_continuation_equals_single_pass():
    """A 32768-token prompt in bucketed chunks (real lengths drawn inside each bucket, padded with
    g = beta = 0), each continuing from the saved fp32 state and conv tail, against the oracle's single
    pass and against the GPU's own single pass."""
    dims = NEXT
    total = 32768
    w, x, rng = make_layer(2, dims, 1, total)
    parts = chunk_lengths(rng, total)
    _say(f"continuation {len(parts)} chunks")
    W = weights(w, dims)
    fills = [{k: rng.standard_normal((1, bucket - n, a.shape[2])).astype(np.float32)
              for k, a in (("m", x.mixed), ("z", x.z), ("a", x.a), ("b", x.b))} for n, bucket in parts]
    ref = oracle.layer_forward(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b)

    def continued(out_f32):
        d = desc_of(dims, out_f32)
        tail = act(np.zeros(dims.tail_shape(1)), dims)
        st = f32(np.zeros(dims.state_shape(1)))
        outs = []
        t0 = 0
        for (n, bucket), fill in zip(parts, fills):
            def pad(a, k):
                return act(np.concatenate([a[:, t0:t0 + n], fill[k]], 1), dims)
            o = gdn.prefill_chunk(d, W, pad(x.mixed, "m"), pad(x.z, "z"), pad(x.a, "a"), pad(x.b, "b"), i32([n]),
                                  tail, st)
            outs.append(host(o[0, :n]))
            t0 += n
        torch.cuda.synchronize()
        return np.concatenate(outs, 0), st, tail

    cont, st, tail = continued(False)
    assert_out_close(cont, ref["out"][0], dims, "continued out vs oracle")
    assert_state_close(host(st[0]), ref["H"][0], "continued state vs oracle")
    np.testing.assert_array_equal(host(tail[0]), ref["tail"][0].astype(np.float32))
    cont32, st32, tail32 = continued(True)
    assert_out_flat(cont32, ref["out"][0], "continued fp32 out vs oracle")
    assert torch.equal(st32, st) and torch.equal(tail32, tail)
    d = desc_of(dims)
    # the GPU's own single pass
    tail1 = act(np.zeros(dims.tail_shape(1)), dims)
    st1 = f32(np.zeros(dims.state_shape(1)))
    o1 = gdn.prefill_chunk(d, W, act(x.mixed, dims), act(x.z, dims), act(x.a, dims), act(x.b, dims), i32([total]),
                           tail1, st1)
    torch.cuda.synchronize()
    assert_out_close(host(o1[0]), ref["out"][0], dims, "single-pass out vs oracle")
    # continued vs single pass: each is within the bound of the oracle, so they differ by at most twice it
    diff = np.abs(cont - host(o1[0]))
    assert np.all(diff <= 2 * (2e-3 + 2.0 ** -8 * np.abs(ref["out"][0]))), float(diff.max())
    assert state_rel_err(host(st1[0]), host(st[0])) <= 2e-3


# ---------------------------------------------------------------------------------------------------
# conv

# the kernel walks 64-token spans in 8-token groups: 203 and 131 tokens end mid-group in a later span
@pytest.mark.parametrize("dims,B,L,lens", [(TINY, 1, 64, [64]), (NEXT, 3, 70, [70, 2, 0]), (SMALL, 2, 33, [33, 17]),
                                           (SMALL, 2, 203, [203, 130]), (NEXT, 3, 131, [131, 1, 64]),
                                           (LayerDims(n_k=2, n_v=4, d_k=32, d_v=128), 2, 100, [100, 37])])
def test_conv_chunk(dims, B, L, lens):
    _say(f"conv B={B} L={L}")
    w, x, rng = make_layer(7, dims, B, L, lens)
    t0 = random_state(rng, dims, B)[1]
    d = desc_of(dims)
    tail = act(t0, dims)
    y = gdn.conv_chunk(d, act(w.conv_w, dims), act(x.mixed, dims), i32(lens), tail)
    torch.cuda.synchronize()
    for s in range(B):
        yr, tr = oracle.conv(w.conv_w, t0[s], x.mixed[s], lens[s])
        assert_out_close(host(y[s]), yr, dims, f"y[{s}]")
        np.testing.assert_array_equal(host(tail[s]), tr.astype(np.float32))


# ---------------------------------------------------------------------------------------------------
# decode, verify, accept, commit, copy

def _saved_states(dims, w, rng, B, prefix=64):
    """Saved states as a seeded random prefix leaves them (oracle run, cast to fp32), and the tails."""
    from gdn_inputs import make_inputs
    x = make_inputs(rng, dims, B, prefix)
    r = oracle.layer_forward(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b)
    tails = r["tail"].astype(np.float32)
    return r["H"].astype(np.float32), tails


def _decode_inputs(dims, rng, B, T):
    from gdn_inputs import make_inputs
    return make_inputs(rng, dims, B, T)


@pytest.mark.parametrize("dims,B", [(NEXT, 8), (SMALL, 4), (LayerDims(n_k=2, n_v=8, d_k=64, d_v=64), 3),
                                    (LayerDims(n_k=2, n_v=8, d_k=128, d_v=128), 5),
                                    (LayerDims(n_k=2, n_v=4, d_k=32, d_v=32, act=ACT_F32), 2),
                                    (LayerDims(n_k=2, n_v=6, d_k=64, d_v=64), 3),
                                    (LayerDims(n_k=1, n_v=8, d_k=128, d_v=128), 4),
                                    (LayerDims(n_k=2, n_v=12, d_k=32, d_v=32, act=ACT_F32), 2),
                                    (LayerDims(n_k=2, n_v=4, d_k=64, d_v=128), 3),
                                    (LayerDims(n_k=2, n_v=8, d_k=128, d_v=32, act=ACT_F32), 2),
                                    (LayerDims(n_k=1, n_v=3, d_k=32, d_v=64), 2)])
@pytest.mark.parametrize("out_f32", [False, True])
def test_decode_step_vs_oracle(dims, B, out_f32):
    _say(f"decode B={B} dims={dims} out_f32={out_f32}")
    w, _, rng = make_layer(8, dims, 1, 1)
    H0, T0 = _saved_states(dims, w, rng, B)
    x = _decode_inputs(dims, rng, B, 1)
    d = desc_of(dims, out_f32)
    # pool with extra rows and a permuted slot map
    npool = B + 3
    slots = rng.permutation(npool)[:B].astype(np.int32)
    poolH = np.zeros(dims.state_shape(npool), np.float32)
    poolT = np.zeros(dims.tail_shape(npool), np.float32)
    poolH[slots], poolT[slots] = H0, T0
    sp, tp = f32(poolH), act(poolT, dims)
    out = gdn.decode_step(d, weights(w, dims), act(x.mixed[:, 0], dims), act(x.z[:, 0], dims), act(x.a[:, 0], dims),
                          act(x.b[:, 0], dims), i32(slots), tp, sp, check_slots=True)
    torch.cuda.synchronize()
    ref = oracle.layer_forward(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, None, T0, H0)
    if out_f32:
        assert out.dtype == torch.float32
        assert_out_flat(host(out), ref["out"][:, 0], "decode fp32 out")
    else:
        assert_out_close(host(out), ref["out"][:, 0], dims)
    hp = host(sp)
    assert_state_close(hp[slots], ref["H"])
    np.testing.assert_array_equal(host(tp)[slots], ref["tail"].astype(np.float32))
    others = np.setdiff1d(np.arange(npool), slots)
    assert np.all(hp[others] == 0)


def test_decode_full_batch_sampled():
    """The decode leg's launch: 256 sequences, 16 key / 32 value heads, d=128, states like the benchmark's;
    sequences 0, 77 and 255 against the oracle, and every output finite."""
    dims, B = NEXT, 256
    _say("decode B=256 (bench launch)")
    w, _, rng = make_layer(61, dims, 1, 1)
    H0, T0 = random_state(rng, dims, B)
    x = _decode_inputs(dims, rng, B, 1)
    d = desc_of(dims)
    sp, tp = f32(H0), act(T0, dims)
    sp32, tp32 = sp.clone(), tp.clone()
    ins = (act(x.mixed[:, 0], dims), act(x.z[:, 0], dims), act(x.a[:, 0], dims), act(x.b[:, 0], dims))
    out = gdn.decode_step(d, weights(w, dims), *ins, None, tp, sp)
    out32 = gdn.decode_step(desc_of(dims, True), weights(w, dims), *ins, None, tp32, sp32)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    assert torch.equal(sp32, sp) and torch.equal(tp32, tp)
    od = oracle.Dims.of(dims)
    for s in (0, 77, 255):
        sl = slice(s, s + 1)
        ref = oracle.layer_forward(od, w, x.mixed[sl], x.z[sl], x.a[sl], x.b[sl], None, T0[sl], H0[sl])
        assert_out_close(host(out[s]), ref["out"][0, 0], dims, f"decode seq {s}")
        assert_out_flat(host(out32[s]), ref["out"][0, 0], f"decode fp32 out seq {s}")
        assert_state_close(host(sp[s]), ref["H"][0], f"decode state {s}")
        np.testing.assert_array_equal(host(tp[s]), ref["tail"][0].astype(np.float32))


def test_verify_paths_full_size_sampled():
    """The tree-verify leg's launch: 64 sequences x 4 paths x (1+4) tokens, 16/32 heads, d=128; sequences
    5 and 63 (every path) against the oracle."""
    dims, B, P, K = NEXT, 64, 4, 4
    T = K + 1
    _say("verify paths B=64 P=4 (bench launch)")
    w, _, rng = make_layer(62, dims, 1, 1)
    H0, T0 = random_state(rng, dims, B)
    x = path_inputs(rng, dims, B, P, T)
    d = desc_of(dims)
    sp, tp = f32(H0), act(T0, dims)
    ins = (act(x.mixed, dims), act(x.z, dims), act(x.a, dims), act(x.b, dims))
    ck_s, ck_t, out = gdn.verify_paths(d, weights(w, dims), *ins, None, tp, sp)
    ck_s32, ck_t32, out32 = gdn.verify_paths(desc_of(dims, True), weights(w, dims), *ins, None, tp, sp)
    torch.cuda.synchronize()
    assert torch.equal(ck_s32, ck_s) and torch.equal(ck_t32, ck_t)
    od = oracle.Dims.of(dims)
    for s in (5, 63):
        sl = slice(s, s + 1)
        ref = oracle.verify_paths(od, w, x.mixed[sl], x.z[sl], x.a[sl], x.b[sl], T0[sl], H0[sl])
        assert_out_close(host(out[s]), ref["out"][0], dims, f"paths out seq {s}")
        assert_out_flat(host(out32[s]), ref["out"][0], f"paths fp32 out seq {s}")
        cks = host(ck_s[s])
        for p in range(P):
            for i in range(T):
                assert_state_close(cks[p, i], ref["ckpt_H"][0, p, i], f"seq {s} path {p} checkpoint {i}")
        np.testing.assert_array_equal(host(ck_t[s]), ref["ckpt_tail"][0].astype(np.float32))


@pytest.mark.parametrize("seed", range(8))
def test_verify_random_shapes_any_length(seed):
    """Seeded shapes through verify with 1 to 9 tokens per sequence (1-64 sequences, permuted pool rows):
    outputs and every checkpoint against the oracle, and bitwise equal to that many decode steps."""
    r = np.random.default_rng(11000 + seed)
    n_k, d_k = int(r.choice([1, 2, 4, 16])), int(r.choice([32, 64, 128]))
    d_v = d_k if r.random() < 0.6 else int(r.choice([32, 64, 128]))
    dims = LayerDims(n_k=n_k, n_v=n_k * int(r.integers(1, 5)), d_k=d_k, d_v=d_v,
                     act=ACT_F32 if r.random() < 0.25 else ACT_BF16)
    B, T = int(r.integers(1, 65)), int(r.integers(1, 10))
    _say(f"verify random seed={seed} B={B} T={T} dims={dims}")
    w, _, rng = make_layer(11500 + seed, dims, 1, 1)
    H0, T0 = random_state(rng, dims, B)
    x = _decode_inputs(dims, rng, B, T)
    npool = B + int(r.integers(0, 5))
    slots = rng.permutation(npool)[:B].astype(np.int32)
    poolH = np.zeros(dims.state_shape(npool), np.float32)
    poolT = np.zeros(dims.tail_shape(npool), np.float32)
    poolH[slots], poolT[slots] = H0, T0
    sp, tp = f32(poolH), act(poolT, dims)
    d, W = desc_of(dims, True), weights(w, dims)
    ins = [act(a, dims) for a in (x.mixed, x.z, x.a, x.b)]
    ck_s, ck_t, out = gdn.verify_with_checkpoints(d, W, *ins, i32(slots), tp, sp)
    torch.cuda.synchronize()
    ref = oracle.verify(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, T0, H0)
    assert_out_flat(host(out), ref["out"], "verify fp32 out")
    cks = host(ck_s)
    for i in range(T):
        assert_state_close(cks[:, i], ref["ckpt_H"][:, i], f"checkpoint {i}")
    np.testing.assert_array_equal(host(ck_t), ref["ckpt_tail"].astype(np.float32))
    sl = torch.as_tensor(slots, device="cuda").long()
    for i in range(T):
        o = gdn.decode_step(d, W, *[a[:, i].contiguous() for a in ins], i32(slots), tp, sp)
        torch.cuda.synchronize()
        assert torch.equal(sp[sl], ck_s[:, i]) and torch.equal(tp[sl], ck_t[:, i]) and torch.equal(o, out[:, i])


def test_verify_checkpoints_and_commit():
    """Verify batch: 64 sequences x (1+4) tokens with per-token checkpoints; accept with m ~ U{0..4};
    restore the checkpoint; compare with the oracle and, bitwise, with repeated GPU decode."""
    dims, B, K = NEXT, 64, 4
    T = K + 1
    _say("verify B=64 K=4")
    w, _, rng = make_layer(9, dims, 1, 1)
    H0, T0 = _saved_states(dims, w, rng, B)
    x = _decode_inputs(dims, rng, B, T)
    drafts, preds, m_true = verify_draws(rng, B, K)
    d = desc_of(dims)
    W = weights(w, dims)
    sp, tp = f32(H0), act(T0, dims)
    mx, zz, aa, bb = act(x.mixed, dims), act(x.z, dims), act(x.a, dims), act(x.b, dims)
    ck_s, ck_t, out = gdn.verify_with_checkpoints(d, W, mx, zz, aa, bb, None, tp, sp)
    ck_s32, ck_t32, out32 = gdn.verify_with_checkpoints(desc_of(dims, True), W, mx, zz, aa, bb, None, tp, sp)
    torch.cuda.synchronize()
    assert np.array_equal(host(sp), H0), "verify modified the pool"
    assert torch.equal(ck_s32, ck_s) and torch.equal(ck_t32, ck_t)
    ref = oracle.verify(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, T0, H0)
    assert_out_close(host(out), ref["out"], dims, "verify out")
    assert_out_flat(host(out32), ref["out"], "verify fp32 out")
    cks = host(ck_s)
    for i in range(T):
        assert_state_close(cks[:, i], ref["ckpt_H"][:, i], f"checkpoint {i}")
    np.testing.assert_array_equal(host(ck_t), ref["ckpt_tail"].astype(np.float32))
    # bitwise against repeated decode on a copy of the pool
    sp2, tp2 = sp.clone(), tp.clone()
    for i in range(T):
        o = gdn.decode_step(d, W, mx[:, i].contiguous(), zz[:, i].contiguous(), aa[:, i].contiguous(),
                            bb[:, i].contiguous(), None, tp2, sp2)
        torch.cuda.synchronize()
        assert torch.equal(sp2, ck_s[:, i]), f"checkpoint {i} differs bitwise from {i + 1} decode calls"
        assert torch.equal(tp2, ck_t[:, i])
        assert torch.equal(o, out[:, i])
    # accept (bit-exact) and commit through the state copy
    m, em, ne, ci = gdn.accept(i32(drafts), i32(preds))
    torch.cuda.synchronize()
    m_ref, em_ref, ne_ref = oracle.accept(drafts, preds)
    np.testing.assert_array_equal(m.cpu().numpy(), m_ref)
    np.testing.assert_array_equal(m_ref, m_true)
    np.testing.assert_array_equal(em.cpu().numpy(), em_ref)
    np.testing.assert_array_equal(ne.cpu().numpy(), ne_ref)
    np.testing.assert_array_equal(ci.cpu().numpy(), np.arange(B) * T + m_ref)
    slots = i32(np.arange(B))
    gdn.state_copy(d, sp, tp, slots, ck_s, ck_t, ci, B)
    torch.cuda.synchronize()
    for s in range(B):
        assert torch.equal(sp[s], ck_s[s, m_ref[s]])
        assert torch.equal(tp[s], ck_t[s, m_ref[s]])
    assert_state_close(host(sp), ref["ckpt_H"][np.arange(B), m_ref])


def test_verify_strong_decays():
    """The step kernel on the prefill test's gate extremes: 8 sequences x 5 tokens from saved states, with
    a = 40 at token 1, a full forget (a = +inf) at token 2 of every other sequence and a = 12 at token 3
    of the rest; checkpoints and outputs against the oracle, and bitwise equal to repeated decode."""
    dims, B, T = LayerDims(n_k=2, n_v=4, d_k=128, d_v=128), 8, 5
    _say("verify strong decays")
    w, _, rng = make_layer(32, dims, 1, 1)
    w.A_log[:] = np.float32(np.log(16.0))
    w.A_log[0] = 0.0
    H0, T0 = _saved_states(dims, w, rng, B)
    x = _decode_inputs(dims, rng, B, T)
    x.a[:, 1] = 40.0
    x.a[::2, 2] = np.inf
    x.a[1::2, 3] = 12.0
    d = desc_of(dims, True)
    W = weights(w, dims)
    sp, tp = f32(H0), act(T0, dims)
    mx, zz, aa, bb = act(x.mixed, dims), act(x.z, dims), act(x.a, dims), act(x.b, dims)
    ck_s, ck_t, out = gdn.verify_with_checkpoints(d, W, mx, zz, aa, bb, None, tp, sp)
    torch.cuda.synchronize()
    ref = oracle.verify(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, T0, H0)
    assert_out_flat(host(out), ref["out"], "verify fp32 out")
    cks = host(ck_s)
    for i in range(T):
        assert_state_close(cks[:, i], ref["ckpt_H"][:, i], f"checkpoint {i}")
    np.testing.assert_array_equal(host(ck_t), ref["ckpt_tail"].astype(np.float32))
    for i in range(T):
        o = gdn.decode_step(d, W, mx[:, i].contiguous(), zz[:, i].contiguous(), aa[:, i].contiguous(),
                            bb[:, i].contiguous(), None, tp, sp)
        torch.cuda.synchronize()
        assert torch.equal(sp, ck_s[:, i]) and torch.equal(tp, ck_t[:, i]) and torch.equal(o, out[:, i])


@pytest.mark.parametrize("dims", [LayerDims(n_k=2, n_v=16, d_k=128, d_v=128), LayerDims(n_k=2, n_v=6, d_k=64, d_v=64),
                                  LayerDims(n_k=2, n_v=4, d_k=128, d_v=64), LayerDims(n_k=2, n_v=6, d_k=32, d_v=128)])
def test_verify_grouped_gqa_ratio(dims):
    """GQA ratios the kernels run in groups (8: four value heads at a time, 3: one), and key and value
    heads of different dims: verify against the oracle, and every checkpoint bitwise equal to repeated
    in-place decode, which only holds if every group reads the conv tail's q and k rows before the last
    group writes them."""
    B, K = 5, 4
    T = K + 1
    _say(f"verify grouped ratio dims={dims}")
    w, _, rng = make_layer(19, dims, 1, 1)
    H0, T0 = _saved_states(dims, w, rng, B)
    x = _decode_inputs(dims, rng, B, T)
    d = desc_of(dims)
    W = weights(w, dims)
    sp, tp = f32(H0), act(T0, dims)
    mx, zz, aa, bb = act(x.mixed, dims), act(x.z, dims), act(x.a, dims), act(x.b, dims)
    ck_s, ck_t, out = gdn.verify_with_checkpoints(d, W, mx, zz, aa, bb, None, tp, sp)
    torch.cuda.synchronize()
    ref = oracle.verify(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, T0, H0)
    assert_out_close(host(out), ref["out"], dims, "verify out")
    cks = host(ck_s)
    for i in range(T):
        assert_state_close(cks[:, i], ref["ckpt_H"][:, i], f"checkpoint {i}")
    np.testing.assert_array_equal(host(ck_t), ref["ckpt_tail"].astype(np.float32))
    sp2, tp2 = sp.clone(), tp.clone()
    for i in range(T):
        o = gdn.decode_step(d, W, mx[:, i].contiguous(), zz[:, i].contiguous(), aa[:, i].contiguous(),
                            bb[:, i].contiguous(), None, tp2, sp2)
        torch.cuda.synchronize()
        assert torch.equal(sp2, ck_s[:, i]), f"checkpoint {i} differs bitwise from {i + 1} decode calls"
        assert torch.equal(tp2, ck_t[:, i])
        assert torch.equal(o, out[:, i])


def test_verify_paths_and_commit():
    """Batch-of-paths verify: 6 sequences x 4 paths x (1+4) tokens from permuted pool rows, against the
    oracle; every row bitwise equal to a single-path verify of its tokens; the winner by the first
    longest accepted prefix (bit-exact) committed through the state copy."""
    dims, B, P, K = NEXT, 6, 4, 4
    T = K + 1
    _say(f"verify paths B={B} P={P} K={K}")
    w, _, rng = make_layer(13, dims, 1, 1)
    H0, T0 = _saved_states(dims, w, rng, B)
    x = path_inputs(rng, dims, B, P, T)
    drafts, preds, _ = verify_path_draws(rng, B, P, K)
    preds[1, 3, :K] = drafts[1, 3]          # a full match on the last path, which the others miss
    preds[1, :3, 0] = drafts[1, :3, 0] + 1
    preds[2, 1:3, :2] = drafts[2, 1:3, :2]  # a tie between paths 1 and 2 ...
    preds[2, 1:3, 2] = drafts[2, 1:3, 2] + 1
    preds[2, 0, 0], preds[2, 3, 0] = drafts[2, 0, 0] + 1, drafts[2, 3, 0] + 1  # ... that no other path beats
    d = desc_of(dims)
    W = weights(w, dims)
    npool = B + 2
    slots = rng.permutation(npool)[:B].astype(np.int32)
    poolH = np.zeros(dims.state_shape(npool), np.float32)
    poolT = np.zeros(dims.tail_shape(npool), np.float32)
    poolH[slots], poolT[slots] = H0, T0
    sp, tp = f32(poolH), act(poolT, dims)
    mx, zz, aa, bb = act(x.mixed, dims), act(x.z, dims), act(x.a, dims), act(x.b, dims)
    ck_s, ck_t, out = gdn.verify_paths(d, W, mx, zz, aa, bb, i32(slots), tp, sp, check_slots=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(sp), poolH), "verify modified the pool"
    ref = oracle.verify_paths(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, T0, H0)
    assert_out_close(host(out), ref["out"], dims, "verify_paths out")
    cks = host(ck_s)
    for p in range(P):
        for i in range(T):
            assert_state_close(cks[:, p, i], ref["ckpt_H"][:, p, i], f"path {p} checkpoint {i}")
    np.testing.assert_array_equal(host(ck_t), ref["ckpt_tail"].astype(np.float32))
    for p in range(1, P):  # the shared first token leaves every path in the same state
        assert torch.equal(ck_s[:, p, 0], ck_s[:, 0, 0]) and torch.equal(out[:, p, 0], out[:, 0, 0])
    # each row bitwise a single-path verify of its tokens
    for p in range(P):
        s1, t1, o1 = gdn.verify_with_checkpoints(d, W, mx[:, p].contiguous(), zz[:, p].contiguous(),
                                                 aa[:, p].contiguous(), bb[:, p].contiguous(), i32(slots), tp, sp)
        torch.cuda.synchronize()
        assert torch.equal(s1, ck_s[:, p]) and torch.equal(t1, ck_t[:, p]) and torch.equal(o1, out[:, p]), f"path {p}"
    # winner and commit
    m, path, em, ne, ci = gdn.accept_paths(i32(drafts), i32(preds))
    torch.cuda.synchronize()
    m_ref, path_ref, em_ref, ne_ref = oracle.accept_paths(drafts, preds)
    assert path_ref[1] == 3 and m_ref[1] == K and path_ref[2] == 1 and m_ref[2] == 2
    np.testing.assert_array_equal(m.cpu().numpy(), m_ref)
    np.testing.assert_array_equal(path.cpu().numpy(), path_ref)
    np.testing.assert_array_equal(em.cpu().numpy(), em_ref)
    np.testing.assert_array_equal(ne.cpu().numpy(), ne_ref)
    np.testing.assert_array_equal(ci.cpu().numpy(), (np.arange(B) * P + path_ref) * T + m_ref)
    gdn.state_copy(d, sp, tp, i32(slots), ck_s, ck_t, ci, B)
    torch.cuda.synchronize()
    for s in range(B):
        assert torch.equal(sp[int(slots[s])], ck_s[s, path_ref[s], m_ref[s]])
        assert torch.equal(tp[int(slots[s])], ck_t[s, path_ref[s], m_ref[s]])


def test_accept_paths_exhaustive():
    """Every pair of paths over a vocabulary of 2 with K = 2, and a random batch of 4 paths with K = 4."""
    import itertools
    K, P = 2, 2
    dr1 = np.array(list(itertools.product(range(2), repeat=K)), np.int32)
    pr1 = np.array(list(itertools.product(range(2), repeat=K + 1)), np.int32)
    one = [(a, b) for a in dr1 for b in pr1]
    pairs = list(itertools.product(range(len(one)), repeat=P))
    D = np.array([[one[i][0] for i in pr] for pr in pairs], np.int32)
    Q = np.array([[one[i][1] for i in pr] for pr in pairs], np.int32)
    rng = np.random.default_rng(31)
    D4, Q4, _ = verify_path_draws(rng, 500, 4, 4, vocab=3)
    for dr, pr in ((D, Q), (D4, Q4)):
        m, path, em, ne, ci = gdn.accept_paths(i32(dr), i32(pr))
        torch.cuda.synchronize()
        m_ref, path_ref, em_ref, ne_ref = oracle.accept_paths(dr, pr)
        np.testing.assert_array_equal(m.cpu().numpy(), m_ref)
        np.testing.assert_array_equal(path.cpu().numpy(), path_ref)
        np.testing.assert_array_equal(em.cpu().numpy(), em_ref)
        np.testing.assert_array_equal(ne.cpu().numpy(), ne_ref)
        Bn, Pn, Kn = dr.shape
        np.testing.assert_array_equal(ci.cpu().numpy(), (np.arange(Bn) * Pn + path_ref) * (Kn + 1) + m_ref)


def test_accept_exhaustive():
    import itertools
    K = 4
    dr = np.array(list(itertools.product(range(3), repeat=K)), np.int32)
    pr = np.array(list(itertools.product(range(3), repeat=K + 1)), np.int32)
    D = np.repeat(dr, len(pr), 0)
    P = np.tile(pr, (len(dr), 1))
    m, em, ne, ci = gdn.accept(i32(D), i32(P))
    torch.cuda.synchronize()
    m_ref, em_ref, ne_ref = oracle.accept(D, P)
    np.testing.assert_array_equal(m.cpu().numpy(), m_ref)
    np.testing.assert_array_equal(em.cpu().numpy(), em_ref)
    np.testing.assert_array_equal(ne.cpu().numpy(), ne_ref)


@pytest.mark.parametrize("dims", [NEXT, LayerDims(n_k=2, n_v=6, d_k=64, d_v=32)])
def test_state_copy_gather_scatter(dims):
    _say(f"state copy dims={dims}")
    d = desc_of(dims)
    rng = np.random.default_rng(10)
    n_src, n_dst, n = 7, 9, 5
    Sx, Tx = random_state(rng, dims, n_src)
    src_s, src_t = f32(Sx), act(Tx, dims)
    dst_s = f32(np.zeros(dims.state_shape(n_dst)))
    dst_t = act(np.zeros(dims.tail_shape(n_dst)), dims)
    si = rng.permutation(n_src)[:n].astype(np.int32)
    di = rng.permutation(n_dst)[:n].astype(np.int32)
    exp_s, exp_t = dst_s.cpu().numpy(), dst_t.view(torch.int16).cpu().numpy()
    oracle.state_copy(exp_s, exp_t, di, src_s.cpu().numpy(), src_t.view(torch.int16).cpu().numpy(), si, n)
    gdn.state_copy(d, dst_s, dst_t, i32(di), src_s, src_t, i32(si), n)
    torch.cuda.synchronize()
    assert dst_s.cpu().numpy().tobytes() == exp_s.tobytes()
    assert dst_t.view(torch.int16).cpu().numpy().tobytes() == exp_t.tobytes()
    # states only, identity indices
    dst2 = f32(np.zeros(dims.state_shape(n_src)))
    gdn.state_copy(d, dst2, None, None, src_s, None, None, n_src)
    torch.cuda.synchronize()
    assert torch.equal(dst2, src_s)


def test_state_zero_rows_and_pools():
    """The state zero: rows idx[i] of both pools, of the state pool alone and of the tail pool alone, and
    every row when idx is NULL; rows not named keep their bits."""
    dims = NEXT
    _say("state zero")
    d = desc_of(dims)
    rng = np.random.default_rng(11)
    S, T = random_state(rng, dims, 9)
    idx = np.array([7, 2, 4], np.int32)
    others = np.setdiff1d(np.arange(9), idx)
    for which in ("both", "state", "tail"):
        sp, tp = f32(S), act(T, dims)
        gdn.state_zero(d, sp if which != "tail" else None, tp if which != "state" else None, i32(idx), 3)
        torch.cuda.synchronize()
        zs, zt = which != "tail", which != "state"
        assert int(torch.count_nonzero(sp[idx.tolist()])) == 0 if zs else torch.equal(sp, f32(S))
        assert int(torch.count_nonzero(tp[idx.tolist()])) == 0 if zt else torch.equal(tp, act(T, dims))
        assert torch.equal(sp[others.tolist()], f32(S)[others.tolist()]) and torch.equal(tp[others.tolist()], act(T, dims)[others.tolist()])
    sp, tp = f32(S), act(T, dims)
    gdn.state_zero(d, sp, tp)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(sp)) == 0 and int(torch.count_nonzero(tp)) == 0


def test_timing_session_names_every_launch():
    """The per-launch timing session sees each kernel a call launches, in order, with its time (256
    tokens: calls of up to 128 take whole heads and no norm pass)."""
    dims = LayerDims(n_k=2, n_v=4, d_k=128, d_v=128)
    _say("timing session: prefill (split heads) then decode")
    w, x, rng = make_layer(5, dims, 1, 256)
    d = desc_of(dims)
    W = weights(w, dims)
    tail = act(np.zeros(dims.tail_shape(1), np.float32), dims)
    st = f32(np.zeros(dims.state_shape(1), np.float32))
    out = torch.empty(1, 256, dims.value_dim, dtype=torch.bfloat16, device="cuda")
    ws = gdn.prefill_workspace(d, 1, 256)
    gdn.timing_begin(16)
    gdn.prefill_chunk(d, W, act(x.mixed, dims), act(x.z, dims), act(x.a, dims), act(x.b, dims), i32(x.lens),
                      tail, st, out, ws)
    gdn.decode_step(d, W, act(x.mixed[:, 0], dims), act(x.z[:, 0], dims), act(x.a[:, 0], dims),
                    act(x.b[:, 0], dims), None, tail, st, torch.empty(1, dims.value_dim, dtype=torch.bfloat16,
                                                                      device="cuda"))
    recs = gdn.timing_end(16)
    assert [n for n, _ in recs] == ["chunk_prep", "state_pass", "norm", "step_decode"]
    assert all(ms > 0 for _, ms in recs)
    with pytest.raises(gdn.GdnError):
        gdn.timing_end(16)  # no open session


def test_continuation_graph_replay_equals_eager():
    """A prompt of bucketed chunks captured once into a HIP graph (torch.cuda.CUDAGraph around the library
    calls): three replays, each after resetting the state and tail eagerly, give the eager run's outputs
    and final state bit for bit."""
    dims, total = NEXT, 4096
    _say("continuation graph replay")
    w, x, rng = make_layer(63, dims, 1, total)
    parts = chunk_lengths(rng, total)
    d = desc_of(dims)
    W = weights(w, dims)
    calls, t0 = [], 0
    for n, bucket in parts:
        def pad(a):
            seg = a[:, t0:t0 + n]
            fill = rng.standard_normal((1, bucket - n, a.shape[2])).astype(np.float32)
            return act(np.concatenate([seg, fill], 1), dims)
        calls.append((pad(x.mixed), pad(x.z), pad(x.a), pad(x.b), i32([n]),
                      torch.empty(1, bucket, dims.value_dim, dtype=torch.bfloat16, device="cuda"), n))
        t0 += n
    ws = gdn.prefill_workspace(d, 1, max(b for _, b in parts))
    tail = torch.zeros(1, 3, dims.conv_dim, dtype=torch.bfloat16, device="cuda")
    state = torch.zeros(1, dims.n_v, dims.d_k, dims.d_v, dtype=torch.float32, device="cuda")

    def run():
        for mx, zz, aa, bb, ln, out, _ in calls:
            gdn.prefill_chunk(d, W, mx, zz, aa, bb, ln, tail, state, out, ws)

    run()
    torch.cuda.synchronize()
    ref_out = [c[5][0, :c[6]].clone() for c in calls]
    ref_state, ref_tail = state.clone(), tail.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        state.zero_()
        tail.zero_()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        state.zero_()
        tail.zero_()
        for c in calls:
            c[5].fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, c in enumerate(calls):
            assert torch.equal(c[5][0, :c[6]], ref_out[i]), f"replay {rep}: chunk {i} output differs"
        assert torch.equal(state, ref_state) and torch.equal(tail, ref_tail), f"replay {rep}: state differs"


def test_speculative_step_graph_replay_equals_eager():
    """One serving step captured once into a HIP graph: verify 1+K tokens from the pool rows, accept on the
    device, commit the accepted checkpoints into the pool by the device-side checkpoint index, then one
    decode step from the committed rows. Before each of three replays the static inputs get new tokens,
    drafts and predictions (eager copies) and the pools their starting rows; every replay matches an eager
    run of the same calls on the same inputs bit for bit (pools, checkpoints, outputs, accepted lengths)."""
    dims, B, K = NEXT, 8, 4
    T = K + 1
    _say("speculative step graph replay")
    w, _, rng = make_layer(64, dims, 1, 1)
    d = desc_of(dims)
    W = weights(w, dims)
    npool = B + 4
    slots = i32(rng.permutation(npool)[:B])
    H0, T0 = random_state(rng, dims, npool)
    pool0_s, pool0_t = f32(H0), act(T0, dims)
    pool_s, pool_t = pool0_s.clone(), pool0_t.clone()

    def draw(seed):
        r = np.random.default_rng(seed)
        x = _decode_inputs(dims, r, B, T + 1)   # the verify tokens, then the token decoded after the commit
        dr = r.integers(0, 3, size=(B, K)).astype(np.int32)
        pr = r.integers(0, 3, size=(B, K + 1)).astype(np.int32)
        return [act(a, dims) for a in (x.mixed, x.z, x.a, x.b)], i32(dr), i32(pr)

    ins0, dr0, pr0 = draw(100)
    mx, zz, aa, bb = [t.clone() for t in ins0]
    drafts, preds = dr0.clone(), pr0.clone()
    ck_s = torch.empty(B, T, dims.n_v, dims.d_k, dims.d_v, dtype=torch.float32, device="cuda")
    ck_t = torch.empty(B, T, 3, dims.conv_dim, dtype=torch.bfloat16, device="cuda")
    out_v = torch.empty(B, T, dims.value_dim, dtype=torch.bfloat16, device="cuda")
    out_d = torch.empty(B, dims.value_dim, dtype=torch.bfloat16, device="cuda")
    vin = [t[:, :T] for t in (mx, zz, aa, bb)]          # views into the static inputs
    din = [t[:, T] for t in (mx, zz, aa, bb)]
    res = {}

    def step():
        gdn.verify_with_checkpoints(d, W, *[v.contiguous() for v in vin], slots, pool_t, pool_s, ck_s, ck_t, out_v)
        m, em, ne, ci = gdn.accept(drafts, preds)
        gdn.state_copy(d, pool_s, pool_t, slots, ck_s, ck_t, ci, B)
        gdn.decode_step(d, W, *[v.contiguous() for v in din], slots, pool_t, pool_s, out_d)
        res.update(m=m, ci=ci)

    def snapshot():
        return [t.clone() for t in (pool_s, pool_t, ck_s, ck_t, out_v, out_d, res["m"], res["ci"])]

    names = ("state pool", "tail pool", "checkpoint states", "checkpoint tails", "verify out", "decode out", "m",
             "checkpoint index")
    refs = []
    for rep in range(3):
        ins, dr, pr = draw(200 + rep)
        for dst, src in zip((mx, zz, aa, bb, drafts, preds), (*ins, dr, pr)):
            dst.copy_(src)
        pool_s.copy_(pool0_s)
        pool_t.copy_(pool0_t)
        step()
        torch.cuda.synchronize()
        refs.append(snapshot())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        ins, dr, pr = draw(200 + rep)
        for dst, src in zip((mx, zz, aa, bb, drafts, preds), (*ins, dr, pr)):
            dst.copy_(src)
        pool_s.copy_(pool0_s)
        pool_t.copy_(pool0_t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, name in zip(snapshot(), refs[rep], names):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager step"
    # the eager steps themselves: accepted lengths as the oracle's accept rule gives them
    for rep in range(3):
        _, dr, pr = draw(200 + rep)
        m_ref = oracle.accept(dr.cpu().numpy(), pr.cpu().numpy())[0]
        assert np.array_equal(refs[rep][6].cpu().numpy(), m_ref), f"step {rep}: m"


def test_split_exchange_graph_replay_equals_eager():
    """Two continued 1100-token calls on 2 sequences of a 16/32-head layer (64 pairs: 32-column slices)
    captured once into a HIP graph. Eagerly the slices exchange their partial row sums (a cooperative
    launch); under capture the library finishes the norm in a separate pass, which never waits. Three
    replays, each after resetting the state, tail and outputs eagerly, give the same bits every time,
    the eager run's final state and tail bit for bit (the norm does not touch them), and its outputs
    within the bound."""
    dims, B, L = NEXT, 2, 1100
    _say("split-head exchange graph replay")
    w, x, rng = make_layer(64, dims, B, 2 * L)
    d = desc_of(dims)
    W = weights(w, dims)
    lens = i32([L, L - 37])
    calls = []
    for i in range(2):
        sl = slice(i * L, (i + 1) * L)
        calls.append((act(x.mixed[:, sl], dims), act(x.z[:, sl], dims), act(x.a[:, sl], dims), act(x.b[:, sl], dims),
                      torch.empty(B, L, dims.value_dim, dtype=torch.bfloat16, device="cuda")))
    ws = gdn.prefill_workspace(d, B, L)
    tail = torch.zeros(B, 3, dims.conv_dim, dtype=torch.bfloat16, device="cuda")
    state = torch.zeros(B, dims.n_v, dims.d_k, dims.d_v, dtype=torch.float32, device="cuda")

    def run():
        for mx, zz, aa, bb, out in calls:
            with prefill_path("two_phase"):
                gdn.prefill_chunk(d, W, mx, zz, aa, bb, lens, tail, state, out, ws)

    gdn.timing_begin(16)
    run()
    assert [n for n, _ in gdn.timing_end(16)] == ["chunk_prep", "state_pass"] * 2  # eagerly: the exchange
    torch.cuda.synchronize()
    eager_out = [torch.cat([c[4][0], c[4][1, :L - 37]]).clone() for c in calls]
    ref_state, ref_tail = state.clone(), tail.clone()
    ref_out = None
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        state.zero_()
        tail.zero_()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        state.zero_()
        tail.zero_()
        for c in calls:
            c[4].fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [torch.cat([c[4][0], c[4][1, :L - 37]]).clone() for c in calls]
        if ref_out is None:
            ref_out = got
            for i in range(2):  # two roundings to bf16 of fp32 values that differ in the last bits: 1 ulp apart
                a, e = host(got[i]), host(eager_out[i])
                assert np.all(np.abs(a - e) <= 2.0 ** -7 * np.maximum(np.abs(a), np.abs(e)) + 1e-6), f"call {i}"
        for i in range(2):
            assert torch.equal(got[i], ref_out[i]), f"replay {rep}: call {i} output differs"
        assert torch.equal(state, ref_state) and torch.equal(tail, ref_tail), f"replay {rep}: state differs"


@pytest.mark.parametrize("B,L", [(6, 300), (2, 1030)])
def test_fused_graph_replay_equals_eager(B, L):
    """The fused prefill captured into a HIP graph (two continued calls): whole heads at 192 units, and
    segment maps, scan and segments at 64 units. Three replays, each after resetting the state, tail and
    outputs eagerly, give the eager run's bits every time (the fused path takes the same launches
    either way and clears nothing with memsets)."""
    dims = NEXT
    _say(f"fused graph replay B={B} L={L}")
    w, x, rng = make_layer(65, dims, B, 2 * L)
    d = desc_of(dims)
    W = weights(w, dims)
    lens = i32([L] + [L - 37] * (B - 1))
    calls = []
    for i in range(2):
        sl = slice(i * L, (i + 1) * L)
        calls.append((act(x.mixed[:, sl], dims), act(x.z[:, sl], dims), act(x.a[:, sl], dims), act(x.b[:, sl], dims),
                      torch.zeros(B, L, dims.value_dim, dtype=torch.bfloat16, device="cuda")))
    with prefill_path("fused"):
        ws = gdn.prefill_workspace(d, B, L)
    tail = torch.zeros(B, 3, dims.conv_dim, dtype=torch.bfloat16, device="cuda")
    state = torch.zeros(B, dims.n_v, dims.d_k, dims.d_v, dtype=torch.float32, device="cuda")

    def run():
        for mx, zz, aa, bb, out in calls:
            with prefill_path("fused"):
                gdn.prefill_chunk(d, W, mx, zz, aa, bb, lens, tail, state, out, ws)

    run()
    torch.cuda.synchronize()
    ref = [c[4].clone() for c in calls], state.clone(), tail.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        state.zero_()
        tail.zero_()
        for c in calls:
            c[4].fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, c in enumerate(calls):
            assert torch.equal(c[4], ref[0][i]), f"replay {rep}: call {i} output differs from eager"
        assert torch.equal(state, ref[1]) and torch.equal(tail, ref[2]), f"replay {rep}: state or tail differs"


@pytest.mark.parametrize("path,dims,B,L,launches", [
    ("fused", SMALL, 1, 4096, ["fused_map", "fused_scan", "fused", "tail"]),  # 16 units: segment maps, scan, segments
    ("fused", NEXT, 1, 4096, ["fused_map", "fused_scan", "fused", "tail"]),   # 32 units
    ("fused", NEXT, 2, 1030, ["fused_map", "fused_scan", "fused", "tail"]),   # 64 units, 17 chunks: 3 segments
    ("fused", NEXT, 2, 700, ["fused", "tail"]),                               # 11 chunks: too short for 3 segments
    (None, NEXT, 8, 512, ["fused", "tail"]),                                  # 256 units: the library's own choice
    (None, NEXT, 6, 300, ["fused", "tail"]),                                  # 192 units
    (None, NEXT, 5, 300, ["chunk_prep", "state_pass"]),                       # 160 units: the two-launch path
])
def test_prefill_fused_launches(path, dims, B, L, launches):
    """Which launches a d = 128 bf16 prefill call makes: the fused kernel with one workgroup per
    (sequence, value head), preceded by the segment maps and the scan where few units run long calls,
    then the conv-tail update; the library takes it from 192 units on."""
    _say(f"fused launches path={path} B={B} L={L} dims={dims}")
    d = desc_of(dims)
    w, x, rng = make_layer(7, dims, B, L)
    tail = act(np.zeros(dims.tail_shape(B), np.float32), dims)
    st = f32(np.zeros(dims.state_shape(B), np.float32))
    gdn.timing_begin(16)
    with prefill_path(path):
        gdn.prefill_chunk(d, weights(w, dims), act(x.mixed, dims), act(x.z, dims), act(x.a, dims), act(x.b, dims),
                          i32(x.lens), tail, st)
    recs = gdn.timing_end(16)
    assert [n for n, _ in recs] == launches


@pytest.mark.parametrize("dims,B,L,launches", [
    (SMALL, 1, 4096, ["chunk_prep", "state_pass", "norm"]),                # 8 slices of 16 columns: norm pass
    (NEXT, 2, 1030, ["chunk_prep", "state_pass"]),                        # 4 slices, >= 1024 tokens: exchange
    (NEXT, 2, 512, ["chunk_prep", "state_pass", "norm"]),                 # 4 slices, a short call: norm pass
    (NEXT, 5, 256, ["chunk_prep", "state_pass"]),                         # 160 pairs: whole heads
])
def test_prefill_norm_mode_launches(dims, B, L, launches, monkeypatch):
    """The two-launch path (GDN_PREFILL_PATH=two_phase): the gated norm is finished by the state pass
    (whole heads, or split heads exchanging row sums on calls of at least 1024 tokens) or by a separate
    norm pass."""
    monkeypatch.setenv("GDN_PREFILL_PATH", "two_phase")
    _say(f"norm mode launches B={B} L={L} dims={dims}")
    d = desc_of(dims)
    w, x, rng = make_layer(7, dims, B, L)
    tail = act(np.zeros(dims.tail_shape(B), np.float32), dims)
    st = f32(np.zeros(dims.state_shape(B), np.float32))
    gdn.timing_begin(16)
    gdn.prefill_chunk(d, weights(w, dims), act(x.mixed, dims), act(x.z, dims), act(x.a, dims), act(x.b, dims),
                      i32(x.lens), tail, st)
    recs = gdn.timing_end(16)
    assert [n for n, _ in recs] == launches
