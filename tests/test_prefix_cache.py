"""The prefix-state cache's bookkeeping (libgdn gdn_pcache_*, host code) against the plain model of the
"qev_fast/statecache.py" page's StateCache in oracle/prefix_cache.py; no GPU needed."""
import numpy as np
import pytest

import gated_delta_rule_44_amd as gdn
from oracle.prefix_cache import PrefixCacheModel


def _rows(rng, count, vocab=50):
    """Rows that share prefixes the way prompts do: a few stems, extended, cut and varied."""
    stems = [rng.integers(0, vocab, size=int(rng.integers(300, 9000))) for _ in range(4)]
    rows = []
    for _ in range(count):
        if rows and rng.random() < 0.15:  # the same prompt again
            rows.append(rows[int(rng.integers(0, len(rows)))])
            continue
        base = stems[int(rng.integers(0, len(stems)))]
        cut = int(rng.integers(1, len(base) + 1))
        ids = np.concatenate([base[:cut], rng.integers(0, vocab, size=int(rng.integers(0, 3000)))])
        if rng.random() < 0.2 and len(ids) > 10:  # a change somewhere inside the shared part
            ids = ids.copy()
            ids[int(rng.integers(0, len(ids)))] = vocab + 1
        p_state = int(rng.integers(0, len(ids) + 1)) if rng.random() < 0.3 else len(ids) - int(rng.integers(0, 40))
        rows.append((ids.astype(np.int32), max(p_state, 0)))
    return rows


@pytest.mark.parametrize("cfg", [dict(slots=6), dict(slots=40), dict(slots=3, stride=512, tail=0),
                                 dict(slots=12, stride=0, tail=16, max_chunk=640), dict(slots=8, align=0, min_prefix=0)])
def test_cache_matches_model(cfg):
    rng = np.random.default_rng(len(str(cfg)))
    model = PrefixCacheModel(cfg["slots"], **{k: v for k, v in cfg.items() if k != "slots"})
    cache = gdn.PrefixStateCache.__new__(gdn.PrefixStateCache)  # bookkeeping only: no GPU pool
    import ctypes
    lib = gdn.load_library()
    h = ctypes.c_void_p()
    args = dict(stride=2048, tail=16, align=64, max_chunk=2048, min_prefix=256)
    args.update({k: v for k, v in cfg.items() if k != "slots"})
    assert lib.gdn_pcache_create(cfg["slots"], args["stride"], args["tail"], args["align"], args["max_chunk"],
                                 args["min_prefix"], ctypes.byref(h)) == 0
    cache._h, cache._lib = h, lib
    slot_of = {}
    for ids, p_state in _rows(rng, 120):
        best, c0, p, bounds, new = model.row(ids, p_state)
        plan = cache.plan(ids, p_state)
        assert (plan["restored"], plan["c0"], plan["p"], plan["bounds"], plan["new"]) == (best, c0, p, bounds, new)
        # slots: a restored checkpoint is where it was stored; live checkpoints never share a slot
        if best >= 0:
            assert plan["restore_slot"] == slot_of[best]
        for num, sl in zip(plan["new"], plan["snap_slot"]):
            assert (num < 0) == (sl < 0)
            if num >= 0:
                slot_of[num] = sl
        live = model.alive()
        assert cache.alive() == live
        assert len({slot_of[k] for k in live}) == len(live) and all(0 <= slot_of[k] < cfg["slots"] for k in live)
    st = cache.stats()
    assert st == {k: model.stats[k] for k in gdn.PCACHE_STATS}
    assert st["rows"] + st["plain"] == 120 and st["hits"] + st["partial"] > 0
    # only rows with a live checkpoint keep their token ids
    assert st["rows_kept"] == model.rows_remembered() <= len(model.alive())


def test_cache_forgets_evicted_rows():
    """Many distinct rows through a 3-slot pool: the cache keeps the ids of at most 3 rows (bounded
    host memory and lookup time however many rows pass)."""
    import ctypes
    lib = gdn.load_library()
    h = ctypes.c_void_p()
    assert lib.gdn_pcache_create(3, 512, 0, 64, 2048, 64, ctypes.byref(h)) == 0
    rng = np.random.default_rng(3)
    info = (ctypes.c_int32 * 4)()
    b = (ctypes.c_int32 * 16)()
    s = (ctypes.c_int32 * 16)()
    st = (ctypes.c_int64 * len(gdn.PCACHE_STATS))()
    for _ in range(300):
        ids = rng.integers(0, 1000, size=int(rng.integers(64, 1500))).astype(np.int32)
        assert lib.gdn_pcache_row(h, ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(ids), len(ids), 16, info,
                                  b, s, None) >= 0
        lib.gdn_pcache_stats(h, st)
        assert st[gdn.PCACHE_STATS.index("rows_kept")] <= 3
    lib.gdn_pcache_destroy(h)


def test_cache_rejects_without_booking():
    """Too little room for the bounds: GDN_EINVAL and nothing booked."""
    import ctypes
    lib = gdn.load_library()
    h = ctypes.c_void_p()
    assert lib.gdn_pcache_create(4, 512, 16, 64, 2048, 0, ctypes.byref(h)) == 0
    ids = np.arange(5000, dtype=np.int32)
    info = (ctypes.c_int32 * 4)()
    b = (ctypes.c_int32 * 2)()
    s = (ctypes.c_int32 * 2)()
    rc = lib.gdn_pcache_row(h, ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 5000, 5000, 2, info, b, s, None)
    assert rc == -1
    st = (ctypes.c_int64 * len(gdn.PCACHE_STATS))()
    lib.gdn_pcache_stats(h, st)
    assert list(st) == [0] * len(gdn.PCACHE_STATS)
    assert lib.gdn_pcache_create(-1, 512, 16, 64, 2048, 0, ctypes.byref(h)) == -1
    lib.gdn_pcache_destroy(h)


@pytest.mark.gpu
def test_prefix_cache_rows_vs_oracle():
    """Rows through the cache's executor (restore or zero, chunked prefill, snapshots) against the oracle's
    cold run of each whole row: a cold row, a row sharing part of it, an exact repeat (a hit at p) and a
    longer row (a partial hit), with chunks cut at max_chunk and an eviction."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import oracle
    from gdn_inputs import LayerDims, make_layer
    from tests.gpu_helpers import act, assert_out_close, assert_state_close, desc_of, host, weights
    print("[case] prefix cache rows", flush=True)
    dims = LayerDims(n_k=2, n_v=4, d_k=128, d_v=128)
    vocab = 97
    w, table, rng = make_layer(41, dims, 1, vocab)  # the projected inputs of each token id
    d = desc_of(dims)
    W = weights(w, dims)
    cache = gdn.PrefixStateCache(d, slots=5, stride=512, tail=16, align=64, max_chunk=256, min_prefix=128)
    A = rng.integers(0, vocab, size=1300).astype(np.int32)
    rows = [(A, 1300), (np.concatenate([A[:900], rng.integers(0, vocab, size=400)]).astype(np.int32), 1300),
            (A, 1300), (np.concatenate([A, rng.integers(0, vocab, size=200)]).astype(np.int32), 1500),
            (rng.integers(0, vocab, size=700).astype(np.int32), 700)]
    expect_c0 = [0, 768, 1280, 1280, 0]
    od = oracle.Dims.of(dims)
    for r, (ids, p_state) in enumerate(rows):
        n = len(ids)
        x = [f[:, ids] for f in (table.mixed, table.z, table.a, table.b)]
        state = torch.empty(1, dims.n_v, dims.d_k, dims.d_v, dtype=torch.float32, device="cuda")
        tail = torch.empty(1, 3, dims.conv_dim, dtype=torch.bfloat16, device="cuda")
        out = torch.zeros(1, n, dims.value_dim, dtype=torch.bfloat16, device="cuda")
        plan = cache.run_row(W, ids, *[act(f, dims) for f in x], state, tail, out, p_state)
        torch.cuda.synchronize()
        assert plan["c0"] == expect_c0[r], (r, plan)
        ref = oracle.layer_forward(od, w, *x)
        c0 = plan["c0"]
        assert_out_close(host(out[0, c0:]), ref["out"][0, c0:], dims, f"row {r} out")
        assert_state_close(host(state[0]), ref["H"][0], f"row {r} state")
        np.testing.assert_array_equal(host(tail[0]), ref["tail"][0].astype(np.float32))
    st = cache.stats()
    assert st["hits"] == 1 and st["partial"] == 2 and st["cold"] == 2 and st["evicted"] > 0
