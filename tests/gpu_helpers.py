"""Shared plumbing for the GPU parity tests: numpy inputs -> device tensors, the tolerance checks, and
canary-guarded buffers.

Tolerances (the layer's stated bar):
  outputs   |gpu - ref| <= 2e-3 on fp32 outputs (out_dtype = GDN_F32, with bf16 activations the output
            before its bf16 rounding): the arithmetic itself is held to the flat bound;
            |gpu - ref| <= 2e-3 + 2^-8 |ref| on bf16 outputs, whose own rounding (half an ulp, 2^-9 |y|
            relative) alone exceeds 2e-3 once |y| > 1;
  states    max |dH| <= 1e-3 * max |H_ref| per (sequence, value head);
  tails, integers, copies: bit-exact.
"""
from __future__ import annotations

import contextlib
import os

import numpy as np
import torch

import gated_delta_rule_44_amd as gdn
from gdn_inputs import ACT_BF16, LayerDims

DEV = "cuda"


def desc_of(d: LayerDims, out_f32: bool = False) -> gdn.GdnDesc:
    return gdn.GdnDesc(n_k=d.n_k, n_v=d.n_v, d_k=d.d_k, d_v=d.d_v, conv_k=d.conv_k,
                       act_dtype=gdn.GDN_BF16 if d.act == ACT_BF16 else gdn.GDN_F32,
                       scale=0.0 if d.scale is None else d.scale, l2_eps=d.l2_eps, rms_eps=d.rms_eps,
                       out_dtype=gdn.GDN_F32 if out_f32 else gdn.GDN_OUT_ACT)


def act(x, d: LayerDims) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))
    return t.to(DEV).to(torch.bfloat16 if d.act == ACT_BF16 else torch.float32).contiguous()


def f32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32))).to(DEV)


def i32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int32))).to(DEV)


def weights(w, d: LayerDims) -> gdn.GdnWeights:
    return gdn.GdnWeights(act(w.conv_w, d), f32(w.A_log), f32(w.dt_bias), f32(w.norm_w))


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def out_excess(gpu: np.ndarray, ref: np.ndarray, d: LayerDims) -> float:
    """Largest amount by which |gpu - ref| exceeds its bound (<= 0 passes)."""
    bound = 2e-3 + (2.0 ** -8) * np.abs(ref) if d.act == ACT_BF16 else 2e-3
    return float(np.max(np.abs(gpu - ref) - bound)) if gpu.size else -1.0


def assert_out_close(gpu: np.ndarray, ref: np.ndarray, d: LayerDims, what="out"):
    ex = out_excess(gpu, ref, d)
    if ex > 0:
        err = np.abs(gpu - ref)
        i = np.unravel_index(np.argmax(err - (2.0 ** -8) * np.abs(ref)), err.shape)
        raise AssertionError(f"{what}: bound exceeded by {ex:.3e}; max err {err.max():.3e} at {i}: "
                             f"gpu={gpu[i]:.6f} ref={ref[i]:.6f}")


def state_rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over (sequence, head) of max|dH| / max|H_ref|; arrays [..., n_v, d_k, d_v]."""
    diff = np.abs(gpu - ref).max(axis=(-1, -2))
    scale = np.maximum(np.abs(ref).max(axis=(-1, -2)), 1e-30)
    return float((diff / scale).max())


def assert_state_close(gpu: np.ndarray, ref: np.ndarray, what="state"):
    e = state_rel_err(gpu, ref)
    assert e <= 1e-3, f"{what}: relative error {e:.3e} > 1e-3"


def assert_out_flat(gpu: np.ndarray, ref: np.ndarray, what="out", bound=2e-3):
    """The flat output bound, for fp32 outputs."""
    if gpu.size == 0:
        return
    err = np.abs(gpu - ref)
    if not np.all(err <= bound):
        i = np.unravel_index(np.nanargmax(np.where(np.isnan(err), np.inf, err)), err.shape)
        raise AssertionError(f"{what}: max |gpu - ref| {np.nanmax(err):.3e} > {bound:g} at {i}: "
                             f"gpu={gpu[i]:.6f} ref={ref[i]:.6f}")


# ---- canary-guarded device buffers: the kernel gets the interior, margins hold a byte pattern ---------

GUARD_BYTES = 4096
GUARD_PATTERN = 0xA5


class Guarded:
    """A device tensor of `shape` with GUARD_BYTES of pattern bytes on either side (the interior starts on
    a 4 KB boundary, so it keeps the alignment of a fresh allocation)."""

    def __init__(self, shape, dtype, fill=None):
        n = int(np.prod(shape))
        esz = torch.tensor([], dtype=dtype).element_size()
        self.nbytes = n * esz
        self.raw = torch.full((2 * GUARD_BYTES + self.nbytes,), GUARD_PATTERN, dtype=torch.uint8, device=DEV)
        self.t = self.raw[GUARD_BYTES:GUARD_BYTES + self.nbytes].view(dtype).view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def check(self, what: str):
        head = self.raw[:GUARD_BYTES]
        tail = self.raw[GUARD_BYTES + self.nbytes:]
        for part, name in ((head, "before"), (tail, "after")):
            bad = torch.nonzero(part != GUARD_PATTERN)
            assert bad.numel() == 0, f"{what}: {bad.numel()} bytes written {name} the buffer"


@contextlib.contextmanager
def prefill_path(path):
    """Force the prefill path (None: the library's own choice; "fused" or "two_phase")."""
    old = os.environ.get("GDN_PREFILL_PATH")
    if path is None:
        os.environ.pop("GDN_PREFILL_PATH", None)
    else:
        os.environ["GDN_PREFILL_PATH"] = path
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("GDN_PREFILL_PATH", None)
        else:
            os.environ["GDN_PREFILL_PATH"] = old


# both prefill paths for d = 128 with bf16 activations (other shapes always take the two-launch path)
BOTH = ("fused", "two_phase")
