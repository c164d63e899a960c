"""Seeded synthetic inputs for the Gated DeltaNet layer (shared by the tests, the bench and smoke()).

This module only draws numbers: it holds none of the layer's arithmetic, so the CPU oracle and the
HIP path can both consume what it produces without sharing any computation. Every tensor that an
activation-dtype buffer will hold is rounded here to the activation precision (bf16 round-to-nearest-
even, or left in fp32), so that both sides read bit-identical values.

Draw order for one layer (seed fixed by the caller; a fresh generator per layer):
    conv_w, A_log, dt_bias, norm_w, mixed, z, a, b, then any workload extras (chunk lengths, drafts).

Distributions (the workload descriptions of the single-layer, chunk-continuation, verify and stack
workloads; the projected inputs are those of the in-projection split in CacheQwen35._gdn of the
qev_fast/statecache.py page, whose order is [mixed qkv | z | b | a]):
    conv_w  ~ N(0, 0.5^2)            [C_ch, K]    (0.5 read as the standard deviation)
    A_log   ~ U(log 1, log 16)       [n_v]        fp32
    dt_bias ~ N(0, 0.1^2)            [n_v]        fp32
    norm_w  = 1 + N(0, 0.1^2)        [d_v]        fp32 (ones would hide the multiply)
    mixed   ~ N(0, 1)                [B, L, C_ch] pre-conv q|k|v channels
    z       ~ N(0, 1)                [B, L, n_v*d_v]
    a, b    ~ N(0, 1)                [B, L, n_v]
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ACT_BF16 = "bf16"
ACT_F32 = "f32"

# chunk buckets of the chunk-continuation workload (a power-of-two subset of the page's bucket list)
CHUNK_BUCKETS = (16, 32, 64, 128, 256, 512, 1024, 2048)


def bf16_round(x) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns float32 holding bf16 values."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out.reshape(x.shape)


def bf16_bits(x) -> np.ndarray:
    """The upper 16 bits of fp32 values that are already bf16-representable (uint16 array)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclass(frozen=True)
class LayerDims:
    n_k: int
    n_v: int
    d_k: int
    d_v: int
    conv_k: int = 4
    act: str = ACT_BF16
    rms_eps: float = 1e-6
    l2_eps: float = 1e-6
    scale: float | None = None  # None: d_k ** -0.5

    @property
    def key_dim(self) -> int:
        return self.n_k * self.d_k

    @property
    def value_dim(self) -> int:
        return self.n_v * self.d_v

    @property
    def conv_dim(self) -> int:
        return 2 * self.key_dim + self.value_dim

    @property
    def kc(self) -> int:
        return self.conv_k - 1

    @property
    def q_scale(self) -> float:
        return float(self.d_k) ** -0.5 if self.scale is None else float(self.scale)

    def state_shape(self, n: int) -> tuple:
        return (n, self.n_v, self.d_k, self.d_v)

    def tail_shape(self, n: int) -> tuple:
        return (n, self.kc, self.conv_dim)


@dataclass
class LayerWeights:
    conv_w: np.ndarray   # [C_ch, K] float32 (bf16 values when act is bf16)
    A_log: np.ndarray    # [n_v] float32
    dt_bias: np.ndarray  # [n_v] float32
    norm_w: np.ndarray   # [d_v] float32


@dataclass
class LayerInputs:
    mixed: np.ndarray    # [B, L, C_ch]
    z: np.ndarray        # [B, L, n_v*d_v]
    a: np.ndarray        # [B, L, n_v]
    b: np.ndarray        # [B, L, n_v]
    lens: np.ndarray     # [B] int32 real lengths
    extras: dict = field(default_factory=dict)


def _act(x: np.ndarray, dims: LayerDims) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return bf16_round(x) if dims.act == ACT_BF16 else x


def make_weights(rng: np.random.Generator, dims: LayerDims) -> LayerWeights:
    conv_w = _act(rng.normal(0.0, 0.5, size=(dims.conv_dim, dims.conv_k)), dims)
    A_log = rng.uniform(np.log(1.0), np.log(16.0), size=dims.n_v).astype(np.float32)
    dt_bias = rng.normal(0.0, 0.1, size=dims.n_v).astype(np.float32)
    norm_w = (1.0 + rng.normal(0.0, 0.1, size=dims.d_v)).astype(np.float32)
    return LayerWeights(conv_w, A_log, dt_bias, norm_w)


def make_inputs(rng: np.random.Generator, dims: LayerDims, B: int, L: int, lens=None) -> LayerInputs:
    mixed = _act(rng.standard_normal(size=(B, L, dims.conv_dim), dtype=np.float32), dims)
    z = _act(rng.standard_normal(size=(B, L, dims.value_dim), dtype=np.float32), dims)
    a = _act(rng.standard_normal(size=(B, L, dims.n_v), dtype=np.float32), dims)
    b = _act(rng.standard_normal(size=(B, L, dims.n_v), dtype=np.float32), dims)
    if lens is None:
        lens = np.full(B, L, dtype=np.int32)
    return LayerInputs(mixed, z, a, b, np.asarray(lens, dtype=np.int32))


def make_layer(seed: int, dims: LayerDims, B: int, L: int, lens=None):
    """Weights then inputs from one generator seeded with `seed`."""
    rng = np.random.default_rng(seed)
    w = make_weights(rng, dims)
    x = make_inputs(rng, dims, B, L, lens)
    return w, x, rng


def random_state(rng: np.random.Generator, dims: LayerDims, n: int, std: float = 0.05):
    """A random fp32 recurrent state and an activation-precision conv tail, for timing-only runs."""
    S = (rng.standard_normal(size=dims.state_shape(n), dtype=np.float32) * np.float32(std)).astype(np.float32)
    tail = _act(rng.standard_normal(size=dims.tail_shape(n), dtype=np.float32), dims)
    return S, tail


def chunk_lengths(rng: np.random.Generator, total: int, buckets=CHUNK_BUCKETS):
    """Split `total` tokens into chunks: a bucket drawn uniformly, a real length drawn uniformly in
    (previous bucket, bucket]; the last chunk is the remainder. Returns [(real_len, bucket), ...]."""
    out = []
    left = total
    while left > 0:
        i = int(rng.integers(0, len(buckets)))
        lo = buckets[i - 1] if i > 0 else 0
        n = int(rng.integers(lo + 1, buckets[i] + 1))
        n = min(n, left)
        bucket = next(bb for bb in buckets if n <= bb)
        out.append((n, bucket))
        left -= n
    return out


def verify_draws(rng: np.random.Generator, B: int, K: int, vocab: int = 1000):
    """Drafts, the accepted-prefix length m ~ U{0..K}, and predictions that agree with the drafts on
    exactly the first m positions (the rest random)."""
    drafts = rng.integers(0, vocab, size=(B, K), dtype=np.int64).astype(np.int32)
    m = rng.integers(0, K + 1, size=B).astype(np.int32)
    preds = rng.integers(0, vocab, size=(B, K + 1), dtype=np.int64).astype(np.int32)
    for i in range(B):
        preds[i, : m[i]] = drafts[i, : m[i]]
        if m[i] < K and preds[i, m[i]] == drafts[i, m[i]]:
            preds[i, m[i]] = (drafts[i, m[i]] + 1) % vocab
    return drafts, preds, m


def verify_path_draws(rng: np.random.Generator, B: int, P: int, K: int, vocab: int = 1000):
    """P candidate paths per sequence: drafts [B,P,K], a prefix length m ~ U{0..K} per path, and
    predictions [B,P,K+1] that agree with that path's drafts on exactly its first m positions."""
    d, p, m = verify_draws(rng, B * P, K, vocab)
    return d.reshape(B, P, K), p.reshape(B, P, K + 1), m.reshape(B, P)


def path_inputs(rng: np.random.Generator, dims: LayerDims, B: int, P: int, T: int) -> LayerInputs:
    """Projected inputs of P paths of T tokens per sequence ([B,P,T,...]); the paths of a sequence share
    their first token (the root every candidate path continues from)."""
    x = make_inputs(rng, dims, B * P, T)
    out = []
    for a in (x.mixed, x.z, x.a, x.b):
        a = a.reshape((B, P) + a.shape[1:]).copy()
        a[:, 1:, 0] = a[:, :1, 0]
        out.append(a)
    return LayerInputs(*out, np.full(B, T, np.int32))


class SpecStream:
    """Synthetic speculative decoding for B sequences: a seeded ground-truth token stream per sequence
    stands for the verifier's greedy continuation, and each draft equals the ground truth at its position
    with probability q (else another token)."""

    def __init__(self, rng: np.random.Generator, B: int, length: int, vocab: int, q: float):
        self.rng, self.vocab, self.q = rng, vocab, q
        self.truth = rng.integers(0, vocab, size=(B, length)).astype(np.int32)
        self.pos = np.zeros(B, np.int64)  # index of each sequence's last emitted token (not yet consumed)

    def draw(self, K: int):
        """-> (x [B], drafts [B,K], preds [B,K+1]) for the next step."""
        B = len(self.pos)
        idx = self.pos[:, None] + np.arange(K + 2)[None, :]
        if idx.max() >= self.truth.shape[1]:
            raise ValueError("ground-truth stream exhausted")
        t = np.take_along_axis(self.truth, idx, axis=1)
        x, preds = t[:, 0], t[:, 1:K + 2]
        drafts = preds[:, :K].copy()
        miss = self.rng.random((B, K)) >= self.q
        drafts[miss] = (drafts[miss] + 1 + self.rng.integers(0, self.vocab - 1, size=int(miss.sum()))) % self.vocab
        return x.astype(np.int32), drafts.astype(np.int32), preds.astype(np.int32)

    def advance(self, m: np.ndarray):
        self.pos += np.asarray(m, np.int64) + 1


# ---- the workloads -----------------------------------------------------------------------------------

TINY = LayerDims(n_k=2, n_v=4, d_k=32, d_v=32, act=ACT_F32)            # T=64, chunk 16
SMALL = LayerDims(n_k=16, n_v=16, d_k=128, d_v=128)                     # 1 x 4096 prefill
NEXT = LayerDims(n_k=16, n_v=32, d_k=128, d_v=128)                      # continuation / verify / stack

WORKLOADS = {
    "tiny": dict(dims=TINY, B=1, T=64, chunk=16),
    "prefill_4k": dict(dims=SMALL, B=1, T=4096, chunk=64),
    "continuation_32k": dict(dims=NEXT, B=1, T=32768, chunk=64),
    "verify_b64_k4": dict(dims=NEXT, B=64, T=5, chunk=64),
    "stack_prefill": dict(dims=NEXT, B=8, T=8192, chunk=64, layers=36),
    "stack_decode": dict(dims=NEXT, B=256, T=1, chunk=64, layers=36),
}
