"""GPU: every entry point at element offsets past 2^31 (byte offsets past 2^32), and at its largest batch.

A few seeded base sequences are tiled over enough batch rows (or pool rows, or checkpoint rows) that the
last rows start beyond 2^31 elements of their buffer. Sequences are independent and every one does the
same arithmetic, so each tiled copy must equal its base bit for bit, wherever it sits; the bases are also
checked against the oracle (fp32 outputs at the flat 2e-3 bound, states at 1e-3 of their largest entry,
conv tails exactly). An offset formed in 32 bits anywhere on the path would read or write the wrong rows
of the far copies. All shapes lie inside the limits include/gdn.h states.

Run on an MI355X: python -u -m pytest tests -m gpu -x -v --timeout 300 --timeout-method thread
"""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_44_amd as gdn
from gdn_inputs import NEXT, LayerDims, make_inputs, make_layer, path_inputs, random_state, verify_draws
from tests.gpu_helpers import (act, assert_out_close, assert_out_flat, assert_state_close, desc_of, f32, host, i32,
                               prefill_path, weights)

pytestmark = pytest.mark.gpu

I32_LIMIT = 2 ** 31


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    gdn.load_library()


@pytest.fixture(autouse=True)
def _release():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _tile(t: torch.Tensor, reps: int) -> torch.Tensor:
    """[K, ...] -> [reps * K, ...], row r holding row r % K"""
    return t.repeat(reps, *([1] * (t.dim() - 1))).contiguous()


def _copies_equal_base(t: torch.Tensor, K: int) -> bool:
    """every row r of t equals row r % K bit for bit (compared as raw bits, so NaN payloads count too)"""
    n = t.shape[0]
    assert n % K == 0
    raw = t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)
    return bool((raw.view(n // K, K, *t.shape[1:]) == raw[:K]).all())


def _prefill_tiled(dims, seed, L, lens, reps):
    """len(lens) seeded base sequences tiled reps times, through both prefill paths (fp32 outputs)"""
    K = len(lens)
    B = K * reps
    w, x, rng = make_layer(seed, dims, K, L, lens)
    H0, t0 = random_state(rng, dims, K)
    od = oracle.Dims.of(dims)
    refs = [oracle.layer_forward(od, w, x.mixed[s:s + 1], x.z[s:s + 1], x.a[s:s + 1], x.b[s:s + 1], x.lens[s:s + 1],
                                 t0[s:s + 1], H0[s:s + 1]) for s in range(K)]
    d = desc_of(dims, out_f32=True)
    W = weights(w, dims)
    ins = [_tile(act(v, dims), reps) for v in (x.mixed, x.z, x.a, x.b)] + [_tile(i32(lens), reps)]
    tail0, st0 = _tile(act(t0, dims), reps), _tile(f32(H0), reps)
    for path in ("fused", "two_phase"):
        _say(f"  path={path}")
        tail, st = tail0.clone(), st0.clone()
        out = torch.zeros(B, L, dims.value_dim, dtype=torch.float32, device="cuda")
        gdn.device_status()  # clear
        with prefill_path(path):
            gdn.prefill_chunk(d, W, *ins, tail, st, out)
        torch.cuda.synchronize()
        assert gdn.device_status() == 0
        for s in range(K):
            n = int(lens[s])
            assert_out_flat(host(out[s, :n]), refs[s]["out"][0, :n], f"out[seq {s}] (path {path})")
            assert_state_close(host(st[s]), refs[s]["H"][0], f"state[seq {s}] (path {path})")
            np.testing.assert_array_equal(host(tail[s]), refs[s]["tail"][0].astype(np.float32))
        # whole rows, those past len included: they carry no meaning, but every copy computes them alike
        for t, name in ((out, "out"), (st, "state"), (tail, "tail")):
            assert _copies_equal_base(t, K), f"{name}: a far copy differs from its base (path {path})"
        del tail, st, out


def test_prefill_past_2g_elements():
    """Prefill on both paths over 2112 sequences of 2048 tokens with 1 key / 2 value heads of 128
    (512 conv channels): the activations of the last sequences start 2.2e9 elements in (4.4 GB)."""
    dims = LayerDims(n_k=1, n_v=2, d_k=128, d_v=128)
    L, reps = 2048, 528
    lens = np.array([2048, 1500, 2047, 65], np.int32)
    B = len(lens) * reps
    assert (B - 1) * L * dims.conv_dim > I32_LIMIT
    _say(f"prefill large offsets B={B} L={L} dims={dims}")
    _prefill_tiled(dims, 71, L, lens, reps)


def test_prefill_max_batch():
    """Prefill at its largest batch, 65535 sequences (1 key / 1 value head of 128, 70 tokens: two chunks,
    ragged, one sequence empty), on both paths."""
    dims = LayerDims(n_k=1, n_v=1, d_k=128, d_v=128)
    lens = np.array([70, 64, 1, 0, 33], np.int32)
    reps = 13107
    assert len(lens) * reps == 65535
    _say(f"prefill max batch B=65535 L=70 dims={dims}")
    _prefill_tiled(dims, 75, 70, lens, reps)


def test_conv_past_2g_elements():
    """The conv over 1056 sequences of 256 tokens at 8192 channels (16 key / 32 value heads of 128): the
    last sequences start 2.2e9 elements in. The bases are checked on every 16th channel."""
    dims = NEXT
    K, L, reps = 4, 256, 264
    B = K * reps
    assert (B - 1) * L * dims.conv_dim > I32_LIMIT
    lens = np.array([256, 100, 1, 0], np.int32)
    _say(f"conv large offsets B={B} L={L}")
    w, x, rng = make_layer(72, dims, K, L, lens)
    t0 = random_state(rng, dims, K)[1]
    d = desc_of(dims)
    tail = _tile(act(t0, dims), reps)
    y = torch.zeros(B, L, dims.conv_dim, dtype=torch.bfloat16, device="cuda")
    gdn.conv_chunk(d, act(w.conv_w, dims), _tile(act(x.mixed, dims), reps), _tile(i32(lens), reps), tail, y)
    torch.cuda.synchronize()
    ch = np.arange(0, dims.conv_dim, 16)  # the conv is depthwise: a channel sample is checked exactly
    for s in range(K):
        yr, tr = oracle.conv(w.conv_w[ch], t0[s][:, ch], x.mixed[s][:, ch], lens[s])
        assert_out_close(host(y[s][:, ch]), yr, dims, f"y[{s}]")
        np.testing.assert_array_equal(host(tail[s])[:, ch], tr.astype(np.float32))
    assert _copies_equal_base(y, K) and _copies_equal_base(tail, K)


def _saved(dims, w, rng, n, prefix=64):
    """states and tails as a seeded 64-token prefix leaves them (oracle), fp32"""
    x = make_inputs(rng, dims, n, prefix)
    r = oracle.layer_forward(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b)
    return r["H"].astype(np.float32), r["tail"].astype(np.float32)


def test_decode_pool_rows_past_2g_elements():
    """Decode from pool rows 4096.. of a 4100-row pool of 16/32 heads (2 MB a row): those rows start
    past 2^31 floats. Bitwise equal to the same step on a 4-row pool, and the oracle's result."""
    dims, B, npool = NEXT, 4, 4100
    per_row = dims.n_v * dims.d_k * dims.d_v
    slots = np.array([4099, 4096, 1, 4097], np.int32)
    assert int(slots.max()) * per_row >= I32_LIMIT
    _say(f"decode large pool npool={npool} slots={slots.tolist()}")
    w, _, rng = make_layer(73, dims, 1, 1)
    H0, T0 = _saved(dims, w, rng, B)
    x = make_inputs(rng, dims, B, 1)
    d = desc_of(dims, out_f32=True)
    W = weights(w, dims)
    step_in = [act(v[:, 0], dims) for v in (x.mixed, x.z, x.a, x.b)]
    sp = torch.zeros(dims.state_shape(npool), dtype=torch.float32, device="cuda")
    tp = torch.zeros(dims.tail_shape(npool), dtype=torch.bfloat16, device="cuda")
    sl = i32(slots).long()
    sp[sl], tp[sl] = f32(H0), act(T0, dims)
    out = gdn.decode_step(d, W, *step_in, i32(slots), tp, sp, check_slots=True)
    sp_small, tp_small = f32(H0), act(T0, dims)
    out_small = gdn.decode_step(d, W, *step_in, None, tp_small, sp_small)
    torch.cuda.synchronize()
    ref = oracle.layer_forward(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, None, T0, H0)
    assert_out_flat(host(out), ref["out"][:, 0], "decode fp32 out")
    assert torch.equal(out, out_small)
    assert torch.equal(sp[sl], sp_small) and torch.equal(tp[sl], tp_small)
    assert_state_close(host(sp_small), ref["H"])
    touched = sp.view(npool, -1).abs().amax(dim=1) != 0
    assert sorted(torch.nonzero(touched).flatten().tolist()) == sorted(slots.tolist()), "rows outside the slots"


def test_verify_checkpoints_past_2g_elements():
    """Verify 832 sequences x 5 tokens of 16/32 heads (the checkpoints of the last ones start past 2^31
    floats, 8.7 GB in all), four base sequences tiled; then accept and commit through the state copy, whose
    sources lie past that offset too."""
    dims, K, reps, T = NEXT, 4, 208, 5
    B = K * reps
    per_row = dims.n_v * dims.d_k * dims.d_v
    assert (B * T - 1) * per_row >= I32_LIMIT
    _say(f"verify large checkpoints B={B} T={T}")
    w, _, rng = make_layer(74, dims, 1, 1)
    H0, T0 = _saved(dims, w, rng, K)
    x = make_inputs(rng, dims, K, T)
    d = desc_of(dims, out_f32=True)
    W = weights(w, dims)
    ins = [_tile(act(v, dims), reps) for v in (x.mixed, x.z, x.a, x.b)]
    sp, tp = _tile(f32(H0), reps), _tile(act(T0, dims), reps)  # pool row b holds base b % 4
    sp0 = sp.clone()
    ck_s, ck_t, out = gdn.verify_with_checkpoints(d, W, *ins, None, tp, sp)
    torch.cuda.synchronize()
    assert torch.equal(sp, sp0), "verify modified the pool"
    del sp0
    ref = oracle.verify(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, T0, H0)
    assert_out_flat(host(out[:K]), ref["out"], "verify fp32 out")
    cks = host(ck_s[:K])
    for i in range(T):
        assert_state_close(cks[:, i], ref["ckpt_H"][:, i], f"checkpoint {i}")
    np.testing.assert_array_equal(host(ck_t[:K]), ref["ckpt_tail"].astype(np.float32))
    for t, name in ((out, "out"), (ck_s, "ckpt_state"), (ck_t, "ckpt_tail")):
        assert _copies_equal_base(t, K), f"{name}: a far copy differs from its base"
    # accept per sequence, then commit every sequence's accepted checkpoint (index b*T + m, up to 4159)
    drafts, preds, _ = verify_draws(rng, B, T - 1)
    m, _, _, ci = gdn.accept(i32(drafts), i32(preds))
    dst_s = torch.zeros(dims.state_shape(B), dtype=torch.float32, device="cuda")
    dst_t = torch.zeros(dims.tail_shape(B), dtype=torch.bfloat16, device="cuda")
    gdn.state_copy(d, dst_s, dst_t, i32(np.arange(B)), ck_s, ck_t, ci, B)
    torch.cuda.synchronize()
    assert int(ci.max()) * per_row >= I32_LIMIT, "no commit source past 2^31 floats"
    src = ci.long()
    assert torch.equal(dst_s, ck_s.view(B * T, *dims.state_shape(1)[1:])[src])
    assert torch.equal(dst_t, ck_t.view(B * T, *dims.tail_shape(1)[1:])[src])


def test_decode_max_batch():
    """Decode at its largest batch, 65535 sequences (1/1 heads of 128), sequence b owning pool row
    65534 - b."""
    dims = LayerDims(n_k=1, n_v=1, d_k=128, d_v=128)
    K, reps = 5, 13107
    B = K * reps
    _say(f"decode max batch B={B}")
    w, _, rng = make_layer(76, dims, 1, 1)
    H0, T0 = _saved(dims, w, rng, K)
    x = make_inputs(rng, dims, K, 1)
    d = desc_of(dims, out_f32=True)
    step_in = [_tile(act(v[:, 0], dims), reps) for v in (x.mixed, x.z, x.a, x.b)]
    slots = np.arange(B - 1, -1, -1, dtype=np.int32)
    sp = _tile(f32(H0), reps).flip(0).contiguous()  # row B-1-b holds base b % K
    tp = _tile(act(T0, dims), reps).flip(0).contiguous()
    out = gdn.decode_step(d, weights(w, dims), *step_in, i32(slots), tp, sp)
    torch.cuda.synchronize()
    ref = oracle.layer_forward(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, None, T0, H0)
    assert_out_flat(host(out[:K]), ref["out"][:, 0], "decode fp32 out")
    sq, tq = sp.flip(0).contiguous(), tp.flip(0).contiguous()  # back to row b = sequence b
    assert_state_close(host(sq[:K]), ref["H"])
    np.testing.assert_array_equal(host(tq[:K]), ref["tail"].astype(np.float32))
    for t, name in ((out, "out"), (sq, "state"), (tq, "tail")):
        assert _copies_equal_base(t, K), f"{name}: a far copy differs from its base"


def test_verify_paths_max_batch():
    """Tree verify at its largest B * P = 65535: 13107 sequences x 5 paths x 2 tokens (1/1 heads of 128),
    three base sequences tiled."""
    dims = LayerDims(n_k=1, n_v=1, d_k=128, d_v=128)
    K, reps, P, T = 3, 4369, 5, 2
    B = K * reps
    assert B * P == 65535
    _say(f"verify paths max batch B={B} P={P} T={T}")
    w, _, rng = make_layer(77, dims, 1, 1)
    H0, T0 = _saved(dims, w, rng, K)
    x = path_inputs(rng, dims, K, P, T)
    d = desc_of(dims, out_f32=True)
    ins = [_tile(act(v, dims), reps) for v in (x.mixed, x.z, x.a, x.b)]
    sp, tp = _tile(f32(H0), reps), _tile(act(T0, dims), reps)
    ck_s, ck_t, out = gdn.verify_paths(d, weights(w, dims), *ins, None, tp, sp)
    torch.cuda.synchronize()
    ref = oracle.verify_paths(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, T0, H0)
    assert_out_flat(host(out[:K]), ref["out"], "paths fp32 out")
    cks = host(ck_s[:K])
    for p in range(P):
        for i in range(T):
            assert_state_close(cks[:, p, i], ref["ckpt_H"][:, p, i], f"path {p} checkpoint {i}")
    np.testing.assert_array_equal(host(ck_t[:K]), ref["ckpt_tail"].astype(np.float32))
    for t, name in ((out, "out"), (ck_s, "ckpt_state"), (ck_t, "ckpt_tail")):
        assert _copies_equal_base(t, K), f"{name}: a far copy differs from its base"


def test_state_copy_and_zero_max_rows():
    """The state copy and the state zero at their largest count, 65535 records (1/1 heads of 128): a
    scatter by a seeded permutation, then zeroing every row through the same index list."""
    dims = LayerDims(n_k=1, n_v=1, d_k=128, d_v=128)
    n = 65535
    _say(f"state copy / zero n={n}")
    d = desc_of(dims)
    gen = torch.Generator(device="cuda").manual_seed(78)
    src_s = torch.randn(dims.state_shape(n), generator=gen, device="cuda")
    src_t = torch.randn(dims.tail_shape(n), generator=gen, device="cuda").to(torch.bfloat16)
    perm = torch.from_numpy(np.random.default_rng(78).permutation(n).astype(np.int32)).cuda()
    dst_s, dst_t = torch.zeros_like(src_s), torch.zeros_like(src_t)
    gdn.state_copy(d, dst_s, dst_t, perm, src_s, src_t, None, n)  # dst row perm[i] <- src row i
    torch.cuda.synchronize()
    assert torch.equal(dst_s[perm.long()], src_s) and torch.equal(dst_t[perm.long()], src_t)
    gdn.state_zero(d, dst_s, dst_t, perm, n)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(dst_s)) == 0 and int(torch.count_nonzero(dst_t)) == 0
