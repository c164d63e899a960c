"""gdn_prefill_chunk_noalloc (the prefill entry point that allocates nothing, for callers that cannot)
against gdn_prefill_chunk with a caller workspace, through the C ABI: two calls in a row on the same
device, the second smaller, each checked to the layer's bounds (fp32 outputs: 2e-3, states: 1e-3 of max |H|
per head) against the workspace call on the same inputs and state, plus the host-side rejection of a
call whose workspace exceeds the scratch."""
import ctypes

import numpy as np
import pytest
import torch

import gated_delta_rule_44_amd as gdn
from gdn_inputs import SMALL, LayerDims, make_layer, random_state
from tests.gpu_helpers import act, assert_out_flat, desc_of, f32, host, i32, state_rel_err, weights

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _call(lib, fn, d, W, ins, lens, tail, st, out, B, L, ws=None):
    cd = d.c()
    cw = gdn._Weights(W.conv_w.data_ptr(), W.A_log.data_ptr(), W.dt_bias.data_ptr(), W.norm_w.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [ctypes.byref(cd), ctypes.byref(cw)] + [_ptr(t) for t in ins] + [_ptr(lens), _ptr(tail), _ptr(st), _ptr(out),
                                                                          B, L]
    if ws is None:
        return fn(*args, stream)
    return fn(*args, _ptr(ws), ws.numel(), stream)


def _case(lib, dims: LayerDims, seed, B, L, lens):
    print(f"[case] no-alloc prefill B={B} L={L} dims={dims}", flush=True)
    w, x, rng = make_layer(seed, dims, B, L, lens)
    H0, t0 = random_state(rng, dims, B)
    d = desc_of(dims, out_f32=True)
    W = weights(w, dims)
    ins = [act(a, dims) for a in (x.mixed, x.z, x.a, x.b)]
    ln = i32(x.lens)
    res = []
    for noalloc in (False, True):
        tail, st = act(t0, dims), f32(H0)
        out = torch.zeros(B, L, dims.value_dim, dtype=torch.float32, device="cuda")
        if noalloc:
            rc = _call(lib, lib.gdn_prefill_chunk_noalloc, d, W, ins, ln, tail, st, out, B, L)
        else:
            ws = gdn.prefill_workspace(d, B, L)
            rc = _call(lib, lib.gdn_prefill_chunk, d, W, ins, ln, tail, st, out, B, L, ws)
        assert rc == 0, lib.gdn_last_error().decode()
        torch.cuda.synchronize()
        res.append((out, st, tail))
    (o1, s1, t1), (o2, s2, t2) = res
    for s in range(B):
        n = int(x.lens[s])
        assert_out_flat(host(o2[s, :n]), host(o1[s, :n]), f"seq {s}: no-alloc vs workspace output")
        assert state_rel_err(host(s2[s]), host(s1[s])) <= 1e-3, f"seq {s}: states differ beyond the bound"
    assert torch.equal(t1, t2), "conv tails differ"


def test_noalloc_prefill_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    lib = gdn.load_library()
    # one 4096-token sequence, 16/16 heads: the two-launch workspace (~140 MB) exceeds the 64 MiB scratch,
    # so the call runs the fused path with segment maps in the scratch
    _case(lib, SMALL, 31, 1, 4096, [4096])
    # then a smaller call on the same scratch: three ragged sequences, 2/4 heads, the two-launch path
    _case(lib, LayerDims(n_k=2, n_v=4, d_k=128, d_v=128), 32, 3, 300, [300, 171, 0])
    # and a smaller one again with key and value heads of different dims (zero-padded copies in the scratch)
    _case(lib, LayerDims(n_k=2, n_v=4, d_k=64, d_v=128), 33, 2, 150, [150, 67])
    # a call whose workspace exceeds the scratch and has no fused path is refused before any launch
    d = desc_of(LayerDims(n_k=16, n_v=64, d_k=64, d_v=64))
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(d.c()), 4, 8192) > (64 << 20)
    p = ctypes.c_void_p(1 << 20)
    cw = gdn._Weights(1 << 20, 1 << 20, 1 << 20, 1 << 20)
    rc = lib.gdn_prefill_chunk_noalloc(ctypes.byref(d.c()), ctypes.byref(cw), p, p, p, p, p, p, p, p, 4, 8192, None)
    assert rc == -1 and b"static scratch" in lib.gdn_last_error()
