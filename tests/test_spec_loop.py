"""The speculative-decoding control loop (gated_delta_rule_44_amd.spec) on the GPU: direct commit from
verify checkpoints, the replay fallback and the commit by row index (then finish()) end in the same pool
bits and emit the same tokens; the pool
after the loop equals the oracle's recurrence over the tokens the loop consumed; the bridge copies pools."""
import numpy as np
import pytest
import torch

import gated_delta_rule_44_amd as gdn
from gated_delta_rule_44_amd import spec
from gdn_inputs import NEXT, SpecStream, make_layer, random_state

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    gdn.load_library()


def test_spec_loop_direct_equals_replay_and_oracle():
    import oracle
    from tests.gpu_helpers import act, assert_state_close, desc_of, f32, host, weights
    print("[case] spec loop B=4 K=4", flush=True)
    dims, B, K, vocab, steps = NEXT, 4, 4, 64, 10
    w, table, rng = make_layer(51, dims, 1, vocab)
    H0, T0 = random_state(rng, dims, B)
    d = desc_of(dims)
    W = weights(w, dims)
    tab = [act(f, dims)[0] for f in (table.mixed, table.z, table.a, table.b)]
    pools = {mode: (f32(H0), act(T0, dims)) for mode in ("direct", "replay", "remap")}
    loops = {mode: spec.SpecDecodeLoop(d, W, tab, K, np.arange(B), *pools[mode], mode=mode) for mode in pools}
    streams = {mode: SpecStream(np.random.default_rng(7), B, 400, vocab, 0.6) for mode in pools}
    for _ in range(steps):
        res = {}
        for mode in ("direct", "replay", "remap"):
            x, dr, pr = streams[mode].draw(K)
            res[mode] = loops[mode].step(x, dr, pr)
            m, em, _ = res[mode]
            for b in range(B):  # emitted = the ground truth after x
                p0 = streams[mode].pos[b]
                np.testing.assert_array_equal(em[b, :m[b] + 1], streams[mode].truth[b, p0 + 1:p0 + m[b] + 2])
            streams[mode].advance(m)
        for mode in ("replay", "remap"):
            np.testing.assert_array_equal(res["direct"][0], res[mode][0])
            assert torch.equal(res["direct"][2], res[mode][2])
    torch.cuda.synchronize()
    assert torch.equal(pools["remap"][0], f32(H0)), "remap wrote the caller's pool before finish()"
    loops["remap"].finish()
    torch.cuda.synchronize()
    for mode in ("replay", "remap"):
        assert torch.equal(pools["direct"][0], pools[mode][0]) and torch.equal(pools["direct"][1], pools[mode][1]), mode
    st = loops["direct"].stats
    pos = streams["direct"].pos
    assert sum(st.accept_hist) == steps * B and st.tokens == int(pos.sum()) and st.direct_commits == steps
    r = loops["replay"].stats
    assert r.fallback_replays == steps and r.replayed_tokens == int(pos.sum()) and r.accept_hist == st.accept_hist
    rep = st.report()
    assert rep.accepted_draft_tokens == st.tokens - steps * B and 0 < rep.acceptance_rate < 1
    # the pool after the loop is the recurrence over the consumed tokens truth[b, :pos_b]
    od = oracle.Dims.of(dims)
    for b in range(B):
        ids = streams["direct"].truth[b, :pos[b]]
        x = [f[:, ids] for f in (table.mixed, table.z, table.a, table.b)]
        ref = oracle.layer_forward(od, w, *x, None, T0[b:b + 1], H0[b:b + 1])
        assert_state_close(host(pools["direct"][0][b]), ref["H"][0], f"sequence {b} state")
        np.testing.assert_array_equal(host(pools["direct"][1][b]), ref["tail"][0].astype(np.float32))


def test_bridge_copies_pools():
    from tests.gpu_helpers import act, desc_of, f32
    dims = NEXT
    d = desc_of(dims)
    rng = np.random.default_rng(3)
    S, Tl = random_state(rng, dims, 5)
    src_s, src_t = f32(S), act(Tl, dims)
    dst_s, dst_t = torch.zeros_like(src_s), torch.zeros_like(src_t)
    rep = spec.bridge(d, dst_s, dst_t, src_s, src_t, 5, seen_tokens=1234)
    assert torch.equal(dst_s, src_s) and torch.equal(dst_t, src_t)
    assert rep.seen_tokens == 1234 and abs(rep.mib - 5 * gdn.state_record_bytes(d) / 2 ** 20) < 1e-9 and rep.seconds > 0
