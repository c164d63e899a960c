"""Benchmark of the Gated DeltaNet layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--only prefill|stack|continuation|decode|verify|verify_paths|prefix_cache|spec_loop|conv|copy|peaks]

Headline (`value`): prefill tokens/s of one layer on one sequence of 4096 tokens, 16 key / 16 value
heads, d_k = d_v = 128, bf16 activations, fp32 state, continued from a saved state (one step = one
gdn_prefill_chunk call: conv, gates, L2 norms, chunked delta rule, gated RMSNorm, state and tail
write-back). Input sets rotate so that the 256 MB last-level cache does not hold the step's inputs.
`ms_per_step` is the median of per-call HIP-event times on the launch stream.

`roofline` is that of the dominant launch of the call, timed live through the library's per-launch
event session (gdn_timing_begin/end) on the launch stream, priced against the dense f16 MFMA peak with
its algorithmic FLOP: the state pass with the inter-chunk step (6 d_k d_v per token and value head),
chunk_prep with the intra-chunk contractions (Gram, W, U', P), the fused launch (the path of shapes
with many (sequence, value head) units, such as the stack layer) with both. `call` prices the whole call: its
algorithmic bytes against HBM (the call's bound: 141 FLOP/B is below the ~312 FLOP/B ridge) and its
algorithmic FLOP against MFMA. `traffic` is the counter-measured HBM bytes of that launch when the
committed counter summary was taken on the current sources, else null.

The same run also measures, each as a sub-object of the one JSON line:
  prefill_stack - one layer of the 9B-like stack: 8 x 8192 tokens, 16 key / 32 value heads
  decode  - 36 GDN layers x 256 sequences x 1 token (one step = 36 gdn_decode_step calls), state GB/s
  verify  - 64 sequences x (1+4) tokens with checkpoints, then accept and the commit copy
  continuation - a 32768-token prompt in bucketed chunks, each continuing from the saved state
  verify_paths - the same with 4 candidate paths per sequence (tree verify), accept over paths, commit
  prefix_cache - 8 rows of 8192 tokens sharing 6144 through the prefix-state cache, against no cache
  spec_loop - the speculative-decoding loop (verify, accept, commit or replay) over 64 sequences
  conv    - the standalone causal conv + SiLU over 8 x 8192 tokens of the stack layer's channels
  copy    - the O(1) state bridge: 256 records {fp32 state, conv tail} of one layer
  measured_peaks - the MFMA probe's dense f16 TFLOP/s and the copy leg's GB/s beside the published peaks
  cpu_baseline - the fp64 oracle on the host cores on the prefill workload; every other leg carries its
                 own, on a bounded sample of its workload scaled to the leg's unit (the sample is
                 stated in each)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0


# ---- device tensors from the seeded numpy inputs --------------------------------------------------------
def _desc(gdn, d):
    from gdn_inputs import ACT_BF16
    return gdn.GdnDesc(n_k=d.n_k, n_v=d.n_v, d_k=d.d_k, d_v=d.d_v, conv_k=d.conv_k,
                       act_dtype=gdn.GDN_BF16 if d.act == ACT_BF16 else gdn.GDN_F32,
                       scale=0.0 if d.scale is None else d.scale, l2_eps=d.l2_eps, rms_eps=d.rms_eps)


def _act(torch, x, d):
    from gdn_inputs import ACT_BF16
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32))).to("cuda")
    return t.to(torch.bfloat16 if d.act == ACT_BF16 else torch.float32).contiguous()


def _f32(torch, x):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32))).to("cuda")


def _i32(torch, x):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int32))).to("cuda")


def _weights(torch, gdn, w, d):
    return gdn.GdnWeights(_act(torch, w.conv_w, d), _f32(torch, w.A_log), _f32(torch, w.dt_bias),
                          _f32(torch, w.norm_w))


class _dev:
    """The helpers above bound to torch and the binding."""

    def __init__(self, torch, gdn):
        self.desc_of = lambda d: _desc(gdn, d)
        self.act = lambda x, d: _act(torch, x, d)
        self.f32 = lambda x: _f32(torch, x)
        self.i32 = lambda x: _i32(torch, x)
        self.weights = lambda w, d: _weights(torch, gdn, w, d)


def prefill_work(dims, T: int, C: int = 64):
    """Algorithmic FLOP and HBM bytes of one prefill call over T tokens of one sequence."""
    nk, nv, dk, dv = dims.n_k, dims.n_v, dims.d_k, dims.d_v
    flop_tok = nv * (2 * C * (dk + 2 * dv) + 6 * dk * dv) + nk * 4 * C * dk
    bytes_tok = 2 * (dims.conv_dim + 2 * nv * dv + 2 * nv)
    bytes_seq = 2 * nv * dk * dv * 4 + 2 * 3 * dims.conv_dim * 2
    return flop_tok * T, bytes_tok * T + bytes_seq


def decode_bytes(dims):
    """HBM bytes of one decode token of one sequence in one layer."""
    return 2 * dims.n_v * dims.d_k * dims.d_v * 4 + 2 * 3 * dims.conv_dim * 2 + 2 * (
        dims.conv_dim + 2 * dims.n_v * dims.d_v + 2 * dims.n_v)


KERNEL_SOURCES = {
    "chunk_prep": ("gdn_prefill.hip", "gdn_common.h", "gdn_kernels.h"),
    "state_pass": ("gdn_prefill.hip", "gdn_common.h", "gdn_kernels.h"),
    "norm": ("gdn_prefill.hip", "gdn_common.h", "gdn_kernels.h"),
    "fused": ("gdn_fused.hip", "gdn_common.h", "gdn_kernels.h"),
    "fused_map": ("gdn_fused.hip", "gdn_common.h", "gdn_kernels.h"),
    "fused_scan": ("gdn_fused.hip", "gdn_common.h", "gdn_kernels.h"),
    "tail": ("gdn_fused.hip", "gdn_common.h", "gdn_kernels.h"),
    "step_decode": ("gdn_step.hip", "gdn_common.h", "gdn_kernels.h"),
    "step_verify": ("gdn_step.hip", "gdn_common.h", "gdn_kernels.h"),
    "copy": ("gdn_state.hip", "gdn_common.h", "gdn_kernels.h"),
    "accept": ("gdn_state.hip", "gdn_common.h", "gdn_kernels.h"),
    "conv": ("gdn_conv.hip", "gdn_common.h", "gdn_kernels.h"),
}


def kernel_hash(kernel=None) -> str:
    """Hash of the sources a kernel is built from (all of csrc when kernel is None)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_44_amd", "csrc")
    files = KERNEL_SOURCES[kernel] if kernel else sorted(os.listdir(csrc))
    for f in files:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, if taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload, {}).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def launch_breakdown(torch, gdn, fn, n):
    """Per-launch durations over n calls of fn, from the library's event-timing session on the launch
    stream; returns {kernel: (launches per call, mean ms per launch)}."""
    torch.cuda.synchronize()
    gdn.timing_begin(64 * n)
    for i in range(n):
        fn(i)
    recs = gdn.timing_end(64 * n)
    per = {}
    for name, ms in recs:
        per.setdefault(name, []).append(ms)
    return {k: (len(v) / n, float(np.mean(v))) for k, v in per.items()}


class Timer:
    """HIP events on the current stream (the stream the library launches on)."""

    def __init__(self, torch, n):
        self.torch = torch
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]

    def run(self, fn, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            s, e = self.ev[i]
            s.record()
            fn(warmup + i)
            e.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = [s.elapsed_time(e) for s, e in self.ev[:steps]]
        return float(np.median(per)), wall * 1e3 / steps


def prefill_kernel_flop(dims, T: int, C: int = 64):
    """Algorithmic FLOP of one prefill call split by the launch that does it. Two-phase path: the
    intra-chunk WY/UT contractions (Gram, W, U', P) in chunk_prep, the inter-chunk state pass (U, O, H)
    in state_pass. Fused path: all of it in the fused launch (its segment maps and scan are extra work,
    not counted)."""
    nk, nv, dk, dv = dims.n_k, dims.n_v, dims.d_k, dims.d_v
    intra = T * (nv * 2 * C * (dk + 2 * dv) + nk * 4 * C * dk)
    inter = T * nv * 6 * dk * dv
    return {"chunk_prep": intra, "state_pass": inter, "fused": intra + inter}


def kernel_roofline(workload, kernel, ms, flop=None, nbytes=None):
    """Roofline object of one launch: algorithmic work per launch over its measured duration."""
    sec = ms / 1e3
    if flop is not None:
        ach = flop / sec / 1e12
        r = {"bound": "mfma", "achieved": ach, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": ach / MFMA_PEAK_TFLOPS, "algorithmic_flop_per_launch": flop}
    else:
        ach = nbytes / sec / 1e9
        r = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": ach / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": nbytes}
    r.update(traffic=measured_traffic(workload, kernel), kernel=kernel, ms_per_launch=ms)
    return r


def _prefill_sets(torch, gdn, dims, B, T, nsets, seed0):
    from gdn_inputs import make_layer, random_state
    H = _dev(torch, gdn)
    act, desc_of, f32, i32, weights = H.act, H.desc_of, H.f32, H.i32, H.weights
    d = desc_of(dims)
    sets = []
    for k in range(nsets):
        w, x, rng = make_layer(seed0 + k, dims, B, T)
        S0, tail0 = random_state(rng, dims, B)
        sets.append(dict(w=weights(w, dims), mixed=act(x.mixed, dims), z=act(x.z, dims), a=act(x.a, dims),
                         b=act(x.b, dims), lens=i32(x.lens), tail=act(tail0, dims), state=f32(S0),
                         out=torch.empty(B, T, dims.value_dim, dtype=torch.bfloat16, device="cuda")))
    ws = gdn.prefill_workspace(d, B, T)  # scratch: one buffer reused by every call, as a caller would

    def step(i):
        s = sets[i % nsets]
        gdn.prefill_chunk(d, s["w"], s["mixed"], s["z"], s["a"], s["b"], s["lens"], s["tail"], s["state"],
                          s["out"], ws)
    return step


def _prefill_measure(torch, gdn, args, dims, B, T, nsets, seed0, workload, steps, warmup):
    step = _prefill_sets(torch, gdn, dims, B, T, nsets, seed0)
    ms_event, ms_wall = Timer(torch, steps).run(step, steps, warmup)
    kern = launch_breakdown(torch, gdn, step, steps)
    flop, nbytes = prefill_work(dims, T)
    flop, nbytes = flop * B, nbytes * B
    kflop = {k: v * B for k, v in prefill_kernel_flop(dims, T).items()}
    sec = ms_event / 1e3
    dominant = max(kern, key=lambda k: kern[k][0] * kern[k][1])
    roof = kernel_roofline(workload, dominant, kern[dominant][1],
                           flop=kflop.get(dominant), nbytes=None if dominant in kflop else nbytes)
    res = {
        "tokens_per_s": B * T / sec, "ms_per_call": ms_event, "ms_wall_per_step": ms_wall,
        "roofline": roof,
        "call": {"hbm_achieved_GBs": nbytes / sec / 1e9, "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBS,
                 "mfma_achieved_TFLOPs": flop / sec / 1e12, "mfma_frac": flop / sec / 1e12 / MFMA_PEAK_TFLOPS,
                 "algorithmic_bytes": nbytes, "algorithmic_flop": flop},
        "kernels_ms": {k: round(v[1], 4) for k, v in kern.items()},
    }
    return res


def bench_prefill(torch, gdn, args):
    from gdn_inputs import SMALL
    T = 4096
    # 7 input sets (7 x 86 MB of inputs, outputs and state, > 512 MiB) rotate past the 256 MB last-level
    # cache; the 171 MB workspace is one scratch buffer reused by every call
    return _prefill_measure(torch, gdn, args, SMALL, 1, T, 7, 100, "prefill_4k", args.steps, args.warmup), SMALL, T


def bench_prefill_stack(torch, gdn, args):
    """One GDN layer of the 9B-like stack: 8 sequences x 8192 tokens, 16 key / 32 value heads."""
    from gdn_inputs import NEXT
    res = _prefill_measure(torch, gdn, args, NEXT, 8, 8192, 2, 400, "prefill_stack_layer",
                           max(3, args.steps // 5), max(1, args.warmup // 2))
    res["workload"] = "one layer of the 36-GDN-layer stack: 8 x 8192 tokens, 16/32 heads, d=128, bf16"
    return res


def bench_decode(torch, gdn, args):
    from gdn_inputs import NEXT, make_layer
    H = _dev(torch, gdn)
    act, desc_of, weights = H.act, H.desc_of, H.weights
    dims = NEXT
    L, B = 36, 256
    d = desc_of(dims)
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    layers = []
    for l in range(L):
        w, x, rng = make_layer(200 + l, dims, B, 1)
        st = torch.empty(B, dims.n_v, dims.d_k, dims.d_v, dtype=torch.float32, device="cuda").normal_(0, 0.05, generator=g)
        tl = torch.empty(B, 3, dims.conv_dim, dtype=torch.float32, device="cuda").normal_(0, 1, generator=g).bfloat16()
        layers.append(dict(w=weights(w, dims), mixed=act(x.mixed[:, 0], dims), z=act(x.z[:, 0], dims),
                           a=act(x.a[:, 0], dims), b=act(x.b[:, 0], dims), tail=tl, state=st,
                           out=torch.empty(B, dims.value_dim, dtype=torch.bfloat16, device="cuda")))

    def step(i):
        for s in layers:
            gdn.decode_step(d, s["w"], s["mixed"], s["z"], s["a"], s["b"], None, s["tail"], s["state"], s["out"])

    steps = max(3, args.steps // 5)
    ms, _ = Timer(torch, steps).run(step, steps, max(1, args.warmup // 2))
    kern = launch_breakdown(torch, gdn, step, 2)
    per_launch = B * decode_bytes(dims)
    roof = kernel_roofline("decode_layer_b256", "step_decode", kern["step_decode"][1], nbytes=per_launch)
    gbs = L * per_launch / (ms / 1e3) / 1e9
    return {"workload": "36 GDN layers x 256 sequences x 1 token, 16/32 heads, d=128, fp32 state",
            "tokens_per_s": B / (ms / 1e3), "ms_per_step": ms, "ms_per_layer": ms / L,
            "GB_per_s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS, "roofline": roof}


def bench_verify(torch, gdn, args):
    from gdn_inputs import NEXT, make_layer, random_state, verify_draws
    H = _dev(torch, gdn)
    act, desc_of, f32, i32, weights = H.act, H.desc_of, H.f32, H.i32, H.weights
    dims = NEXT
    B, K = 64, 4
    T = K + 1
    d = desc_of(dims)
    w, x, rng = make_layer(300, dims, B, T)
    S0, tail0 = random_state(rng, dims, B)
    drafts, preds, _ = verify_draws(rng, B, K)
    W = weights(w, dims)
    pools = [(f32(S0), act(tail0, dims)) for _ in range(3)]  # 3 x 128 MiB rotate past the LLC
    mx, zz, aa, bb = act(x.mixed, dims), act(x.z, dims), act(x.a, dims), act(x.b, dims)
    ck_s = torch.empty(B, T, dims.n_v, dims.d_k, dims.d_v, dtype=torch.float32, device="cuda")
    ck_t = torch.empty(B, T, 3, dims.conv_dim, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(B, T, dims.value_dim, dtype=torch.bfloat16, device="cuda")
    dr, pr = i32(drafts), i32(preds)
    slots = i32(np.arange(B))

    def step(i):
        sp, tp = pools[i % len(pools)]
        gdn.verify_with_checkpoints(d, W, mx, zz, aa, bb, None, tp, sp, ck_s, ck_t, out)
        _, _, _, ci = gdn.accept(dr, pr)
        gdn.state_copy(d, sp, tp, slots, ck_s, ck_t, ci, B)

    ms, _ = Timer(torch, args.steps).run(step, args.steps, args.warmup)
    kern = launch_breakdown(torch, gdn, step, 4)
    rec = dims.n_v * dims.d_k * dims.d_v * 4
    tail_b = 3 * dims.conv_dim * 2
    io = B * T * 2 * (dims.conv_dim + 2 * dims.value_dim + 2 * dims.n_v)
    verify_bytes = B * (rec * (1 + T) + T * tail_b) + io
    nbytes = verify_bytes + B * 2 * (rec + tail_b)
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"workload": "64 sequences x (1+4) tokens, 16/32 heads, d=128: verify + accept + commit",
            "ms_per_step": ms, "tokens_per_s": B * T / (ms / 1e3), "GB_per_s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes,
            "roofline": kernel_roofline("verify_b64_k4", "step_verify", kern["step_verify"][1], nbytes=verify_bytes),
            "kernels_ms": {k: round(v[1], 4) for k, v in kern.items()}}


def bench_verify_paths(torch, gdn, args):
    from gdn_inputs import NEXT, make_layer, path_inputs, random_state, verify_path_draws
    H = _dev(torch, gdn)
    act, desc_of, f32, i32, weights = H.act, H.desc_of, H.f32, H.i32, H.weights
    dims = NEXT
    B, P, K = 64, 4, 4
    T = K + 1
    d = desc_of(dims)
    w, _, rng = make_layer(301, dims, 1, 1)
    x = path_inputs(rng, dims, B, P, T)
    S0, tail0 = random_state(rng, dims, B)
    drafts, preds, _ = verify_path_draws(rng, B, P, K)
    W = weights(w, dims)
    pools = [(f32(S0), act(tail0, dims)) for _ in range(3)]  # 3 x 128 MiB rotate past the LLC
    mx, zz, aa, bb = act(x.mixed, dims), act(x.z, dims), act(x.a, dims), act(x.b, dims)
    ck_s = torch.empty(B, P, T, dims.n_v, dims.d_k, dims.d_v, dtype=torch.float32, device="cuda")
    ck_t = torch.empty(B, P, T, 3, dims.conv_dim, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(B, P, T, dims.value_dim, dtype=torch.bfloat16, device="cuda")
    dr, pr = i32(drafts), i32(preds)
    slots = i32(np.arange(B))

    def step(i):
        sp, tp = pools[i % len(pools)]
        gdn.verify_paths(d, W, mx, zz, aa, bb, None, tp, sp, ck_s, ck_t, out)
        ci = gdn.accept_paths(dr, pr)[4]
        gdn.state_copy(d, sp, tp, slots, ck_s, ck_t, ci, B)

    ms, _ = Timer(torch, args.steps).run(step, args.steps, args.warmup)
    kern = launch_breakdown(torch, gdn, step, 4)
    rec = dims.n_v * dims.d_k * dims.d_v * 4
    tail_b = 3 * dims.conv_dim * 2
    io = B * P * T * 2 * (dims.conv_dim + 2 * dims.value_dim + 2 * dims.n_v)
    verify_bytes = B * (rec + tail_b) + B * P * T * (rec + tail_b) + io  # shared state read once per sequence
    nbytes = verify_bytes + B * 2 * (rec + tail_b)
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"workload": "64 sequences x 4 paths x (1+4) tokens, 16/32 heads, d=128: verify + accept + commit",
            "ms_per_step": ms, "tokens_per_s": B * P * T / (ms / 1e3), "GB_per_s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes,
            "roofline": kernel_roofline("verify_paths_b64_p4_k4", "step_verify", kern["step_verify"][1],
                                        nbytes=verify_bytes),
            "kernels_ms": {k: round(v[1], 4) for k, v in kern.items()}}


def bench_continuation(torch, gdn, args):
    """A 32768-token prompt in bucketed chunks (16/32 heads, d=128): each chunk one gdn_prefill_chunk call
    padded to its bucket, continuing from the previous call's fp32 state and conv tail. Throughput counts
    real tokens only."""
    from gdn_inputs import NEXT, chunk_lengths, make_layer
    H = _dev(torch, gdn)
    act, desc_of, i32, weights = H.act, H.desc_of, H.i32, H.weights
    dims, total = NEXT, 32768
    d = desc_of(dims)
    w, x, rng = make_layer(304, dims, 1, total)
    W = weights(w, dims)
    parts = chunk_lengths(rng, total)
    calls, t0 = [], 0
    for n, bucket in parts:
        def pad(a):
            seg = a[:, t0:t0 + n]
            fill = rng.standard_normal((1, bucket - n, a.shape[2])).astype(np.float32)
            return act(np.concatenate([seg, fill], 1), dims)
        calls.append((pad(x.mixed), pad(x.z), pad(x.a), pad(x.b), i32([n]),
                      torch.empty(1, bucket, dims.value_dim, dtype=torch.bfloat16, device="cuda")))
        t0 += n
    ws = gdn.prefill_workspace(d, 1, max(b for _, b in parts))
    tail = torch.zeros(1, 3, dims.conv_dim, dtype=torch.bfloat16, device="cuda")
    state = torch.zeros(1, dims.n_v, dims.d_k, dims.d_v, dtype=torch.float32, device="cuda")

    def step(i):
        for mx, zz, aa, bb, ln, out in calls:
            gdn.prefill_chunk(d, W, mx, zz, aa, bb, ln, tail, state, out, ws)

    reps = max(2, args.steps // 10)
    ms, _ = Timer(torch, reps).run(step, reps, 1)
    # the same calls captured once into a HIP graph and replayed (the library allocates nothing and never
    # synchronises inside a call, so a caller can capture it)
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cs):
            step(0)
    torch.cuda.current_stream().wait_stream(cs)
    ms_g, _ = Timer(torch, reps).run(lambda i: g.replay(), reps, 1)
    padded = sum(b for _, b in parts)
    # each call's time on its own, by bucket, and a straight-line fit ms = fixed + per_token * bucket
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
    for (e0, e1), (mx, zz, aa, bb, ln, out) in zip(ev, calls):
        e0.record()
        gdn.prefill_chunk(d, W, mx, zz, aa, bb, ln, tail, state, out, ws)
        e1.record()
    torch.cuda.synchronize()
    call_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    by = {}
    for (_, bucket), t in zip(parts, call_ms):
        by.setdefault(bucket, []).append(t)
    per_tok, fixed = np.polyfit([b for _, b in parts], call_ms, 1)
    # roofline of the dominant launch over the prompt: its algorithmic work on the real tokens per launch
    kern = launch_breakdown(torch, gdn, step, 1)
    kflop, nbytes = {}, 0
    for n, _ in parts:
        for k, v in prefill_kernel_flop(dims, n).items():
            kflop[k] = kflop.get(k, 0) + v
        nbytes += prefill_work(dims, n)[1]
    dominant = max(kern, key=lambda k: kern[k][0] * kern[k][1])
    launches = kern[dominant][0]
    roof = kernel_roofline("continuation_32k", dominant, kern[dominant][1],
                           flop=kflop[dominant] / launches if dominant in kflop else None,
                           nbytes=None if dominant in kflop else nbytes / launches)
    flop = sum(kflop[k] for k in ("chunk_prep", "state_pass"))
    sec = ms / 1e3
    return {"workload": "1 x 32768 tokens in %d bucketed chunks, 16/32 heads, d=128" % len(parts),
            "ms_per_prompt": ms, "tokens_per_s": total / sec, "chunks": len(parts),
            "padded_tokens": padded, "ms_per_chunk": ms / len(parts),
            "graph": {"ms_per_prompt": ms_g, "tokens_per_s": total / (ms_g / 1e3)},
            "roofline": roof,
            "call": {"hbm_achieved_GBs": nbytes / sec / 1e9, "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBS,
                     "mfma_achieved_TFLOPs": flop / sec / 1e12, "mfma_frac": flop / sec / 1e12 / MFMA_PEAK_TFLOPS,
                     "algorithmic_bytes": nbytes, "algorithmic_flop": flop},
            "ms_per_call_by_bucket": {str(k): round(float(np.mean(v)), 4) for k, v in sorted(by.items())},
            "calls_by_bucket": {str(k): len(v) for k, v in sorted(by.items())},
            "fit_ms_per_call": {"fixed": float(fixed), "per_bucket_token": float(per_tok)},
            "kernels_ms": {k: round(v[1], 4) for k, v in kern.items()}}


def bench_prefix_cache(torch, gdn, args):
    """Rows of 8192 tokens that share a 6144-token prefix (a system prompt) and differ in their last 2048,
    through the prefix-state cache (restore, 2048-token chunks, snapshots) and through the plain path
    (every row from zero). Throughput counts every row token, computed or reused."""
    from gdn_inputs import NEXT, make_layer
    H = _dev(torch, gdn)
    act, desc_of, weights = H.act, H.desc_of, H.weights
    dims = NEXT
    rows_n, n, shared, vocab = 8, 8192, 6144, 512
    d = desc_of(dims)
    w, table, rng = make_layer(302, dims, 1, vocab)
    W = weights(w, dims)
    tab = [act(f, dims)[0] for f in (table.mixed, table.z, table.a, table.b)]  # per token id
    stem = rng.integers(0, vocab, size=shared)
    rows = [np.concatenate([stem, rng.integers(0, vocab, size=n - shared)]).astype(np.int32) for _ in range(rows_n)]
    inputs = [[t[torch.as_tensor(r, device="cuda").long()][None].contiguous() for t in tab] for r in rows]
    state = torch.empty(1, dims.n_v, dims.d_k, dims.d_v, dtype=torch.float32, device="cuda")
    tail = torch.empty(1, 3, dims.conv_dim, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(1, n, dims.value_dim, dtype=torch.bfloat16, device="cuda")

    def run(cached):
        cache = gdn.PrefixStateCache(d, slots=16, min_prefix=256 if cached else n + 1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for r, x in zip(rows, inputs):
            cache.run_row(W, r, *x, state, tail, out, shared)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3, cache.stats()

    run(True), run(False)  # warm-up
    ms_c, st = min((run(True) for _ in range(max(1, args.steps // 10))), key=lambda r: r[0])
    ms_p, _ = min((run(False) for _ in range(max(1, args.steps // 10))), key=lambda r: r[0])
    tok = rows_n * n
    return {"workload": "8 rows x 8192 tokens sharing a 6144-token prefix, 16/32 heads, d=128, one layer",
            "ms_cached": ms_c, "ms_plain": ms_p, "tokens_per_s_cached": tok / (ms_c / 1e3),
            "tokens_per_s_plain": tok / (ms_p / 1e3), "speedup": ms_p / ms_c, "stats": st}


def bench_spec_loop(torch, gdn, args):
    """The speculative-decoding loop (verify + accept + commit per step, the host reading m back each
    step) over 64 sequences with K = 4 and drafts that match the synthetic verifier with probability 0.7,
    committing verify checkpoints directly, committing them by row index (one copy back into the pool at
    the end, timed), and, for comparison, replaying the accepted prefix."""
    from gated_delta_rule_44_amd import spec
    from gdn_inputs import NEXT, SpecStream, make_layer, random_state
    H = _dev(torch, gdn)
    act, desc_of, f32, weights = H.act, H.desc_of, H.f32, H.weights
    dims, B, K, vocab, steps = NEXT, 64, 4, 1024, 24
    d = desc_of(dims)
    w, table, rng = make_layer(303, dims, 1, vocab)
    W = weights(w, dims)
    tab = [act(f, dims)[0] for f in (table.mixed, table.z, table.a, table.b)]
    S0, tail0 = random_state(rng, dims, B)
    res = {}
    for mode in ("direct", "remap", "replay"):
        sp, tp = f32(S0), act(tail0, dims)
        loop = spec.SpecDecodeLoop(d, W, tab, K, np.arange(B), sp, tp, mode=mode)
        stream = SpecStream(np.random.default_rng(9), B, 8 * steps * (K + 1), vocab, 0.7)
        for _ in range(3):  # warm-up steps
            stream.advance(loop.step(*stream.draw(K))[0])
        loop.stats = spec.LoopStats(K, B)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            stream.advance(loop.step(*stream.draw(K))[0])
        loop.finish()
        torch.cuda.synchronize()
        sec = time.perf_counter() - t0
        res[mode] = {"tokens_per_s": loop.stats.tokens / sec, "ms_per_step": sec / steps * 1e3,
                     "acceptance_rate": loop.stats.report().acceptance_rate, **loop.stats.as_dict()}
    return {"workload": "64 sequences, K=4 drafts per step, synthetic drafts matching with p=0.7, 24 steps, one layer",
            **res}


def bench_conv(torch, gdn, args):
    """The standalone causal conv + SiLU (gdn_conv_chunk) over the stack layer's inputs: 8 x 8192 tokens
    of 8192 bf16 channels, with the conv tail rolled forward. Algorithmic bytes: mixed read once, y
    written once, tails read and written."""
    from gdn_inputs import NEXT
    H = _dev(torch, gdn)
    desc_of = H.desc_of
    dims, B, L = NEXT, 8, 8192
    d = desc_of(dims)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    C = dims.conv_dim
    sets = [torch.empty(B, L, C, device="cuda").normal_(generator=g).bfloat16() for _ in range(2)]
    w = torch.empty(C, 4, device="cuda").normal_(0, 0.5, generator=g).bfloat16()
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    tail = torch.zeros(B, 3, C, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(B, L, C, dtype=torch.bfloat16, device="cuda")

    def step(i):
        gdn.conv_chunk(d, w, sets[i % 2], lens, tail, y)

    ms, _ = Timer(torch, args.steps).run(step, args.steps, args.warmup)
    nbytes = 2 * B * L * C * 2 + 2 * B * 3 * C * 2 + C * 4 * 2
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"workload": "8 x 8192 tokens x 8192 bf16 channels (16/32 heads, d=128)", "ms_per_call": ms,
            "GB_per_s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
            "roofline": kernel_roofline("conv_8x8192", "conv", ms, nbytes=nbytes)}


def bench_copy(torch, gdn, args):
    from gdn_inputs import NEXT
    H = _dev(torch, gdn)
    desc_of = H.desc_of
    dims = NEXT
    n = 256
    d = desc_of(dims)
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    src = [(torch.empty(n, dims.n_v, dims.d_k, dims.d_v, device="cuda").normal_(generator=g),
            torch.empty(n, 3, dims.conv_dim, device="cuda").normal_(generator=g).bfloat16()) for _ in range(2)]
    dst = [(torch.empty_like(s), torch.empty_like(t)) for s, t in src]

    def step(i):
        (ss, st), (ds, dt) = src[i % 2], dst[i % 2]
        gdn.state_copy(d, ds, dt, None, ss, st, None, n)

    ms, _ = Timer(torch, args.steps).run(step, args.steps, args.warmup)
    nbytes = 2 * n * gdn.state_record_bytes(d)
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"workload": "256 state records (fp32 state + bf16 conv tail) of one 16/32-head layer",
            "ms_per_call": ms, "mib": nbytes / 2 / 2 ** 20, "GB_per_s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
            "roofline": kernel_roofline("state_copy_256", "copy", ms, nbytes=nbytes)}


def _best_time(fn, reps):
    best = None
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        dt = time.perf_counter() - t0
        best = dt if best is None else min(best, dt)
    return best


def _cpu(value, unit, threads, sample, seconds, **extra):
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle", "sample": sample,
            "seconds": seconds, **extra}


def cpu_prefill_stack():
    """The oracle on one of the stack layer's 8 sequences (8192 tokens, 16/32 heads, saved state): the
    leg's rate is tokens/s of one layer, and the sequences are independent, so the sample's rate is it."""
    import oracle
    from gdn_inputs import NEXT, make_layer, random_state
    dims, T = NEXT, 8192
    w, x, rng = make_layer(400, dims, 1, T)
    S0, tail0 = random_state(rng, dims, 1)
    th = oracle.default_threads()
    sec = _best_time(lambda: oracle.layer_forward(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, tail=tail0,
                                                  H=S0, threads=th), 1)
    return _cpu(T / sec, "tokens/s", th, "1 of the 8 sequences of one layer (8192 tokens), tokens/s of the sample",
                sec)


def cpu_decode():
    """The oracle's decode step (one token from a saved state and conv tail) for the 256 sequences in 1 of
    the 36 layers, scaled to the whole step (x 36)."""
    import oracle
    from gdn_inputs import NEXT, make_layer, random_state
    dims, B, L, nb = NEXT, 256, 36, 256
    w, x, rng = make_layer(200, dims, nb, 1)
    S0, tail0 = random_state(rng, dims, nb)
    th = oracle.default_threads()
    sec = _best_time(lambda: oracle.layer_forward(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, tail=tail0,
                                                  H=S0, threads=th), 2)
    step = sec * (B / nb) * L
    return _cpu(B / step, "tokens/s", th, "256 sequences x 1 of 36 layers, scaled x36", sec,
                ms_per_step=step * 1e3, GB_per_s=L * B * decode_bytes(dims) / step / 1e9)


def cpu_verify():
    """The oracle's verify (1+4 tokens per sequence, token by token, every checkpoint kept), accept, and
    the commit of the accepted checkpoint, for the 64 sequences."""
    import oracle
    from gdn_inputs import NEXT, make_layer, random_state, verify_draws
    dims, B, nb, K = NEXT, 64, 64, 4
    w, x, rng = make_layer(300, dims, nb, K + 1)
    S0, tail0 = random_state(rng, dims, nb)
    drafts, preds, _ = verify_draws(rng, nb, K)
    th = oracle.default_threads()

    def run():
        r = oracle.verify(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, tail0, S0, threads=th)
        m = oracle.accept(drafts, preds)[0]
        return r["ckpt_H"][np.arange(nb), m].copy(), r["ckpt_tail"][np.arange(nb), m].copy()

    sec = _best_time(run, 2)
    step = sec * B / nb
    return _cpu(B * (K + 1) / step, "tokens/s", th, "64 sequences x (1+4) tokens", sec,
                ms_per_step=step * 1e3)


def cpu_verify_paths():
    """The oracle's tree verify (4 paths x (1+4) tokens from each sequence's state), accept over paths
    and the commit, for 16 of the 64 sequences, scaled x4."""
    import oracle
    from gdn_inputs import NEXT, make_layer, path_inputs, random_state, verify_path_draws
    dims, B, nb, P, K = NEXT, 64, 16, 4, 4
    w, _, rng = make_layer(301, dims, 1, 1)
    x = path_inputs(rng, dims, nb, P, K + 1)
    S0, tail0 = random_state(rng, dims, nb)
    drafts, preds, _ = verify_path_draws(rng, nb, P, K)
    th = oracle.default_threads()

    def run():
        r = oracle.verify_paths(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, tail0, S0, threads=th)
        m, path = oracle.accept_paths(drafts, preds)[:2]
        return r["ckpt_H"][np.arange(nb), path, m].copy()

    sec = _best_time(run, 2)
    step = sec * B / nb
    return _cpu(B * P * (K + 1) / step, "tokens/s", th, "16 of 64 sequences x 4 paths x (1+4) tokens, scaled x4",
                sec, ms_per_step=step * 1e3)


def cpu_continuation():
    """The oracle over an 8192-token prompt of the same recipe (chunk lengths drawn from the same buckets),
    each call continuing from the previous call's state and conv tail, real tokens only."""
    import oracle
    from gdn_inputs import NEXT, chunk_lengths, make_layer
    dims, total = NEXT, 8192
    w, x, rng = make_layer(304, dims, 1, total)
    parts = chunk_lengths(rng, total)
    th = oracle.default_threads()
    od = oracle.Dims.of(dims)

    def run():
        t0, tail, H = 0, None, None
        for n, _ in parts:
            sl = slice(t0, t0 + n)
            r = oracle.layer_forward(od, w, x.mixed[:, sl], x.z[:, sl], x.a[:, sl], x.b[:, sl], tail=tail, H=H,
                                     threads=th)
            tail, H, t0 = r["tail"], r["H"], t0 + n
        return t0

    t0 = time.perf_counter()
    ntok = run()
    sec = time.perf_counter() - t0
    return _cpu(ntok / sec, "tokens/s", th, "an %d-token prompt in %d bucketed chunks (the 32768-token recipe, cut)"
                % (ntok, len(parts)), sec)


def cpu_conv():
    """The oracle's conv + SiLU (one thread) on one of the leg's 8 sequences (8192 tokens x 8192
    channels): the sequences are independent, so the sample's GB/s is the leg's rate."""
    import oracle
    from gdn_inputs import bf16_round
    T, Cs, C, B = 8192, 8192, 8192, 8
    rng = np.random.default_rng(5)
    x = bf16_round(rng.standard_normal((T, Cs), dtype=np.float32))
    w = bf16_round(rng.normal(0.0, 0.5, size=(Cs, 4)).astype(np.float32))
    tail = np.zeros((3, Cs), np.float32)
    sec = _best_time(lambda: oracle.conv(w, tail, x, T), 1)
    nbytes = 2 * T * Cs * 2 + 2 * 3 * Cs * 2 + Cs * 4 * 2
    full = 2 * B * T * C * 2 + 2 * B * 3 * C * 2 + C * 4 * 2
    return _cpu(nbytes / sec / 1e9, "GB/s", 1, "1 of the 8 sequences (8192 tokens x 8192 channels)", sec,
                ms_per_call=sec * full / nbytes * 1e3)


def cpu_copy():
    """The oracle's state record copy (numpy, one thread) of the leg's 256 records of one layer."""
    import oracle
    from gdn_inputs import NEXT
    dims, n = NEXT, 256
    rng = np.random.default_rng(6)
    src_s = rng.standard_normal(dims.state_shape(n), dtype=np.float32)
    src_t = rng.integers(0, 1 << 16, size=dims.tail_shape(n), dtype=np.uint16)  # bf16 bit patterns
    dst_s, dst_t = np.empty_like(src_s), np.empty_like(src_t)
    sec = _best_time(lambda: oracle.state_copy(dst_s, dst_t, None, src_s, src_t, None, n), 2)
    nbytes = 2 * (src_s.nbytes + src_t.nbytes)
    return _cpu(nbytes / sec / 1e9, "GB/s", 1, "the whole leg (256 records)", sec, ms_per_call=sec * 1e3)


def cpu_prefix_cache():
    """The oracle over what the oracle's prefix-cache model plans for the leg's 8 rows (restores, chunk
    ends, snapshots): the whole leg, cached; tokens/s counts every row token, computed or reused."""
    import oracle
    from gdn_inputs import NEXT, make_layer
    from oracle.prefix_cache import PrefixCacheModel
    dims = NEXT
    rows_n, n, shared, vocab = 8, 8192, 6144, 512
    w, table, rng = make_layer(302, dims, 1, vocab)
    stem = rng.integers(0, vocab, size=shared)
    rows = [np.concatenate([stem, rng.integers(0, vocab, size=n - shared)]).astype(np.int32) for _ in range(rows_n)]
    th = oracle.default_threads()
    od = oracle.Dims.of(dims)

    def run():
        model = PrefixCacheModel(16, min_prefix=256)
        snaps = {}
        for ids in rows:
            x = [f[0][ids][None] for f in (table.mixed, table.z, table.a, table.b)]
            ck, c0, _, ends, made = model.row(ids, shared)
            tail, H = snaps[ck] if ck >= 0 else (None, None)
            for e, num in zip(list(ends) + [n], list(made) + [-1]):
                sl = slice(c0, e)
                r = oracle.layer_forward(od, w, *[a[:, sl] for a in x], tail=tail, H=H, threads=th)
                tail, H, c0 = r["tail"], r["H"], e
                if num >= 0:
                    snaps[num] = (tail, H)
            alive = set(model.alive())
            snaps = {k: v for k, v in snaps.items() if k in alive}

    t0 = time.perf_counter()
    run()
    sec = time.perf_counter() - t0
    return _cpu(rows_n * n / sec, "tokens/s", th, "the whole leg, cached (8 rows x 8192 tokens sharing 6144)", sec)


def cpu_spec_loop():
    """The oracle driving the leg's loop in direct-commit mode (verify 1+4 tokens of 64 sequences from the
    token table, accept, keep the accepted checkpoint) for 4 steps of the same seeded draft stream."""
    import oracle
    from gdn_inputs import NEXT, SpecStream, make_layer, random_state
    dims, B, K, vocab, steps = NEXT, 64, 4, 1024, 4
    w, table, rng = make_layer(303, dims, 1, vocab)
    H, tail = random_state(rng, dims, B)
    stream = SpecStream(np.random.default_rng(9), B, 8 * steps * (K + 1), vocab, 0.7)
    th = oracle.default_threads()
    od = oracle.Dims.of(dims)
    emitted = 0
    t0 = time.perf_counter()
    for _ in range(steps):
        x, drafts, preds = stream.draw(K)
        ids = np.concatenate([x[:, None], drafts], 1)
        r = oracle.verify(od, w, *[f[0][ids] for f in (table.mixed, table.z, table.a, table.b)], tail, H, threads=th)
        m = oracle.accept(drafts, preds)[0]
        H, tail = r["ckpt_H"][np.arange(B), m], r["ckpt_tail"][np.arange(B), m]
        stream.advance(m)
        emitted += int((m + 1).sum())
    sec = time.perf_counter() - t0
    return _cpu(emitted / sec, "tokens/s", th, "4 direct-commit steps of the leg's loop (64 sequences, K=4)", sec,
                ms_per_step=sec / steps * 1e3)


def cpu_baseline():
    """The oracle (fp64, OpenMP over value heads) on the prefill workload, on the host cores."""
    import oracle
    from gdn_inputs import SMALL, make_layer
    dims = SMALL
    T = 4096
    w, x, rng = make_layer(100, dims, 1, T)
    threads = oracle.default_threads()
    best = None
    for _ in range(2):
        t0 = time.perf_counter()
        oracle.layer_forward(oracle.Dims.of(dims), w, x.mixed, x.z, x.a, x.b, threads=threads)
        dt = time.perf_counter() - t0
        best = dt if best is None else min(best, dt)
    return {"value": T / best, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "the whole prefill workload (1 x 4096 tokens, 16/16 heads, d=128), best of 2 runs",
            "seconds": best}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="all")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_44_amd as gdn
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    gdn.load_library()
    only = args.only

    line = {"metric": "GDN layer prefill tokens/s (% MFMA peak); decode state GB/s (% HBM peak)",
            "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic"}
    if only in ("all", "prefill"):
        pre, dims, T = bench_prefill(torch, gdn, args)
        line.update(value=pre["tokens_per_s"], ms_per_step=pre["ms_per_call"])
        line["config"] = {"workload": "prefill_4k: 1 sequence x 4096 tokens, 16 key / 16 value heads, d=128",
                          "global_batch": 1, "seq_len": T, "chunk": 64, "parallelism": "single GPU"}
        line["roofline"] = pre["roofline"]
        line["call"] = pre["call"]
        line["kernels_ms"] = pre["kernels_ms"]
        line["ms_wall_per_step"] = pre["ms_wall_per_step"]
    if only in ("all", "stack"):
        line["prefill_stack"] = bench_prefill_stack(torch, gdn, args)
        torch.cuda.empty_cache()
    if only in ("all", "decode"):
        line["decode"] = bench_decode(torch, gdn, args)
        torch.cuda.empty_cache()
    if only in ("all", "verify"):
        line["verify"] = bench_verify(torch, gdn, args)
    if only in ("all", "verify_paths"):
        line["verify_paths"] = bench_verify_paths(torch, gdn, args)
    if only in ("all", "continuation"):
        line["continuation"] = bench_continuation(torch, gdn, args)
    if only in ("all", "prefix_cache"):
        line["prefix_cache"] = bench_prefix_cache(torch, gdn, args)
    if only in ("all", "spec_loop"):
        line["spec_loop"] = bench_spec_loop(torch, gdn, args)
    if only in ("all", "conv"):
        line["conv"] = bench_conv(torch, gdn, args)
    if only in ("all", "copy"):
        line["copy"] = bench_copy(torch, gdn, args)
    if only in ("all", "peaks"):
        # the peaks the rooflines are quoted against, re-derived on this GPU: dense f16 MFMA from the
        # probe kernel (best of 5), HBM streaming from the state-copy leg when it ran
        tf = max(gdn.mfma_probe() for _ in range(5))
        line["measured_peaks"] = {"mfma_f16_TFLOPs": tf, "mfma_frac_of_published": tf / MFMA_PEAK_TFLOPS,
                                  "hbm_copy_GBs": line.get("copy", {}).get("GB_per_s"),
                                  "published": {"mfma_bf16_f16_TFLOPs": MFMA_PEAK_TFLOPS, "hbm_GBs": HBM_PEAK_GBS}}
    if not args.no_cpu:
        # the oracle on the host cores beside each leg that has one (bounded samples, scaled as stated)
        if only in ("all", "prefill"):
            line["cpu_baseline"] = cpu_baseline()
        for leg, fn in (("prefill_stack", cpu_prefill_stack), ("decode", cpu_decode), ("verify", cpu_verify),
                        ("verify_paths", cpu_verify_paths), ("continuation", cpu_continuation),
                        ("prefix_cache", cpu_prefix_cache), ("spec_loop", cpu_spec_loop), ("conv", cpu_conv),
                        ("copy", cpu_copy)):
            if leg in line:
                line[leg]["cpu_baseline"] = fn()
    line["kernel_hash"] = kernel_hash()
    print(json.dumps(line))


if __name__ == "__main__":
    main()
