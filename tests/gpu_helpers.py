"""Shared plumbing for the GPU parity tests: numpy inputs -> device tensors, and the tolerance checks.

Tolerances (the layer's stated bar, read for bf16 outputs):
  outputs   |gpu - ref| <= 2e-3 + 2^-8 |ref| for bf16 outputs (the second term is the output's own
            half-ulp rounding), <= 2e-3 for fp32 outputs;
  states    max |dH| <= 1e-3 * max |H_ref| per (sequence, value head);
  tails, integers, copies: bit-exact.
"""
from __future__ import annotations

import numpy as np
import torch

import gated_delta_rule_44_amd as gdn
from gdn_inputs import ACT_BF16, LayerDims

DEV = "cuda"


def desc_of(d: LayerDims) -> gdn.GdnDesc:
    return gdn.GdnDesc(n_k=d.n_k, n_v=d.n_v, d_k=d.d_k, d_v=d.d_v, conv_k=d.conv_k,
                       act_dtype=gdn.GDN_BF16 if d.act == ACT_BF16 else gdn.GDN_F32,
                       scale=0.0 if d.scale is None else d.scale, l2_eps=d.l2_eps, rms_eps=d.rms_eps)


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
