"""Gated DeltaNet (gated delta-rule) layer hot path for MI355X: Python binding of libgdn.so.

Argument marshalling only. Every step of the layer runs in the HIP kernels behind the C ABI declared
in include/gdn.h; torch provides device memory and the current stream. There is no fallback: if
libgdn.so is missing or the device is not a HIP GPU, the calls raise.

Entry points (same names as the C ABI, without the gdn_ prefix):
    conv_chunk, prefill_workspace_bytes, prefill_chunk, decode_step, verify_with_checkpoints,
    accept, state_copy, state_record_bytes
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_LIBRARY names another build of the same library (the host-sanitizer build of the CPU tests)
LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(_HERE, "libgdn.so")

GDN_BF16 = 0
GDN_F32 = 1
GDN_OUT_ACT = 0          # out in the activation dtype
GDN_STATUS_RANGE = 1     # device status bit: a prefill's final state left the f16 operand range
GDN_STATUS_EXCHANGE = 2  # device status bit: a row-sum exchange wait expired (rows written as NaN)
_ACT_TORCH = {GDN_BF16: torch.bfloat16, GDN_F32: torch.float32}

_STATUS = {0: "GDN_OK", -1: "GDN_EINVAL", -2: "GDN_EUNSUPPORTED", -3: "GDN_EHIP"}


class GdnError(RuntimeError):
    def __init__(self, name: str, code: int, msg: str):
        super().__init__(f"{name} -> {_STATUS.get(code, code)}: {msg}")
        self.code = code


class GdnUnsupported(GdnError):
    """The library has no kernel for this shape (the caller's plain path should take it)."""


class _Desc(ctypes.Structure):
    _fields_ = [("n_k", ctypes.c_int32), ("n_v", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("conv_k", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("l2_eps", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("out_dtype", ctypes.c_int32)]


class _Weights(ctypes.Structure):
    _fields_ = [("conv_w", ctypes.c_void_p), ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
                ("norm_w", ctypes.c_void_p)]


_lib = None
EXPORTS = ("gdn_last_error", "gdn_version", "gdn_conv_chunk", "gdn_prefill_workspace_bytes", "gdn_prefill_chunk",
           "gdn_decode_step", "gdn_verify_with_checkpoints", "gdn_verify_paths", "gdn_accept", "gdn_accept_paths",
           "gdn_state_copy",
           "gdn_state_record_bytes", "gdn_state_zero", "gdn_pcache_create", "gdn_pcache_destroy", "gdn_pcache_row",
           "gdn_pcache_stats", "gdn_pcache_alive", "gdn_mfma_probe", "gdn_timing_begin", "gdn_timing_end",
           "gdn_device_status", "gdn_prefill_chunk_noalloc")


def load_library(path: str = LIB_PATH):
    """Load libgdn.so (built by gated_delta_rule_44_amd.build). Raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m gated_delta_rule_44_amd.build` first")
    lib = ctypes.CDLL(path)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    D = ctypes.POINTER(_Desc)
    W = ctypes.POINTER(_Weights)
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_version.restype = ctypes.c_char_p
    lib.gdn_conv_chunk.argtypes = [D, P, P, P, P, P, I, I, P]
    lib.gdn_prefill_workspace_bytes.argtypes = [D, I, I]
    lib.gdn_prefill_workspace_bytes.restype = Z
    lib.gdn_prefill_chunk.argtypes = [D, W, P, P, P, P, P, P, P, P, I, I, P, Z, P]
    lib.gdn_prefill_chunk_noalloc.argtypes = [D, W, P, P, P, P, P, P, P, P, I, I, P]
    lib.gdn_prefill_chunk_noalloc.restype = I
    lib.gdn_decode_step.argtypes = [D, W, P, P, P, P, P, P, P, P, I, P]
    lib.gdn_verify_with_checkpoints.argtypes = [D, W, P, P, P, P, I, P, P, P, P, P, P, I, P]
    lib.gdn_verify_paths.argtypes = [D, W, P, P, P, P, I, I, P, P, P, P, P, P, I, P]
    lib.gdn_accept.argtypes = [P, P, I, I, P, P, P, P, P]
    lib.gdn_accept_paths.argtypes = [P, P, I, I, I, P, P, P, P, P, P]
    lib.gdn_state_copy.argtypes = [D, P, P, P, P, P, P, I, P]
    lib.gdn_state_record_bytes.argtypes = [D]
    lib.gdn_state_record_bytes.restype = Z
    lib.gdn_state_zero.argtypes = [D, P, P, P, I, P]
    L = ctypes.c_int64
    lib.gdn_pcache_create.argtypes = [I, I, I, I, I, I, ctypes.POINTER(P)]
    lib.gdn_pcache_destroy.argtypes = [P]
    lib.gdn_pcache_destroy.restype = None
    lib.gdn_pcache_row.argtypes = [P, ctypes.POINTER(ctypes.c_int32), I, I, I, ctypes.POINTER(ctypes.c_int32),
                                   ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(L)]
    lib.gdn_pcache_stats.argtypes = [P, ctypes.POINTER(L)]
    lib.gdn_pcache_alive.argtypes = [P, I, ctypes.POINTER(L)]
    lib.gdn_mfma_probe.argtypes = [P, I, I, P]
    lib.gdn_device_status.argtypes = [I, P]
    lib.gdn_device_status.restype = I
    lib.gdn_timing_begin.argtypes = [I]
    lib.gdn_timing_end.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float), I]
    for name in ("gdn_conv_chunk", "gdn_prefill_chunk", "gdn_decode_step", "gdn_verify_with_checkpoints",
                 "gdn_verify_paths", "gdn_accept", "gdn_accept_paths", "gdn_state_copy", "gdn_state_zero",
                 "gdn_pcache_create", "gdn_pcache_row", "gdn_pcache_stats", "gdn_pcache_alive"):
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def version() -> str:
    return load_library().gdn_version().decode()


def device_status(clear: bool = True) -> int:
    """Bits the kernels raised on the current device since the word was last cleared (synchronizes the
    current stream): GDN_STATUS_RANGE = a prefill's final state left the f16 operand range."""
    lib = load_library()
    rc = lib.gdn_device_status(1 if clear else 0, _stream())
    if rc < 0:
        _check("gdn_device_status", rc)
    return rc


@dataclass(frozen=True)
class GdnDesc:
    n_k: int
    n_v: int
    d_k: int
    d_v: int
    conv_k: int = 4
    act_dtype: int = GDN_BF16
    scale: float = 0.0      # <= 0: d_k ** -0.5
    l2_eps: float = 1e-6
    rms_eps: float = 1e-6
    out_dtype: int = GDN_OUT_ACT  # or GDN_F32: fp32 outputs (with bf16 activations, before bf16 rounding)

    @property
    def conv_dim(self) -> int:
        return 2 * self.n_k * self.d_k + self.n_v * self.d_v

    @property
    def kc(self) -> int:
        return self.conv_k - 1

    @property
    def act(self) -> torch.dtype:
        return _ACT_TORCH[self.act_dtype]

    @property
    def out(self) -> torch.dtype:
        """dtype of the layer output"""
        return torch.float32 if self.out_dtype == GDN_F32 else self.act

    def c(self) -> _Desc:
        return _Desc(self.n_k, self.n_v, self.d_k, self.d_v, self.conv_k, self.act_dtype, self.scale, self.l2_eps,
                     self.rms_eps, self.out_dtype)


@dataclass
class GdnWeights:
    conv_w: torch.Tensor   # [C_ch, conv_k] act dtype
    A_log: torch.Tensor    # [n_v] fp32
    dt_bias: torch.Tensor  # [n_v] fp32
    norm_w: torch.Tensor   # [d_v] fp32


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, shape, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise RuntimeError(f"{name}: expected a torch tensor")
    if t.device.type != "cuda":
        raise RuntimeError(f"{name}: must live on the GPU, got {t.device}")
    if device is not None and t.device != device:
        raise RuntimeError(f"{name}: on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise RuntimeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise RuntimeError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _opt(t, name, shape, dtype, device):
    return None if t is None else _dev(t, name, shape, dtype, device)


def _check(name: str, rc: int):
    if rc != 0:
        msg = load_library().gdn_last_error().decode()
        raise (GdnUnsupported if rc == -2 else GdnError)(name, rc, msg)


def _weights(desc: GdnDesc, w: GdnWeights, device) -> _Weights:
    return _Weights(_dev(w.conv_w, "conv_w", (desc.conv_dim, desc.conv_k), desc.act, device).value,
                    _dev(w.A_log, "A_log", (desc.n_v,), torch.float32, device).value,
                    _dev(w.dt_bias, "dt_bias", (desc.n_v,), torch.float32, device).value,
                    _dev(w.norm_w, "norm_w", (desc.d_v,), torch.float32, device).value)


def _check_index(t: torch.Tensor, name: str, hi: int, distinct: bool):
    """Host-side range check of a device index array (one small copy)."""
    h = t.detach().cpu()
    if h.numel() and (int(h.min()) < 0 or int(h.max()) >= hi):
        raise ValueError(f"{name}: values must lie in [0, {hi})")
    if distinct and h.numel() != torch.unique(h).numel():
        raise ValueError(f"{name}: values must be distinct")


def conv_chunk(desc: GdnDesc, conv_w, mixed, lens, conv_tail, y=None):
    """Causal conv + SiLU over [conv_tail | mixed]; conv_tail updated in place. Returns y."""
    lib = load_library()
    B, Lb, C = mixed.shape
    dev = mixed.device
    if y is None:
        y = torch.empty_like(mixed)
    args = (_dev(conv_w, "conv_w", (C, desc.conv_k), desc.act, dev),
            _dev(mixed, "mixed", (B, Lb, desc.conv_dim), desc.act, dev),
            _dev(lens, "lens", (B,), torch.int32, dev),
            _dev(conv_tail, "conv_tail", (B, desc.kc, desc.conv_dim), desc.act, dev),
            _dev(y, "y", (B, Lb, desc.conv_dim), desc.act, dev))
    _check("gdn_conv_chunk", lib.gdn_conv_chunk(ctypes.byref(desc.c()), *args, B, Lb, _stream()))
    return y


def prefill_workspace_bytes(desc: GdnDesc, B: int, Lb: int) -> int:
    return int(load_library().gdn_prefill_workspace_bytes(ctypes.byref(desc.c()), B, Lb))


def prefill_workspace(desc: GdnDesc, B: int, Lb: int, device="cuda") -> torch.Tensor:
    n = prefill_workspace_bytes(desc, B, Lb)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def prefill_chunk(desc: GdnDesc, w: GdnWeights, mixed, z, a, b, lens, conv_tail, state, out=None, ws=None):
    """One padded chunk per sequence through the layer from the saved (conv_tail, state), both updated
    in place. Returns out [B, Lb, n_v*d_v]."""
    lib = load_library()
    B, Lb, _ = mixed.shape
    dev = mixed.device
    nvd = desc.n_v * desc.d_v
    if out is None:
        out = torch.empty(B, Lb, nvd, dtype=desc.out, device=dev)
    if ws is None:
        ws = prefill_workspace(desc, B, Lb, dev)
    cw = _weights(desc, w, dev)
    args = (_dev(mixed, "mixed", (B, Lb, desc.conv_dim), desc.act, dev),
            _dev(z, "z", (B, Lb, nvd), desc.act, dev),
            _dev(a, "a", (B, Lb, desc.n_v), desc.act, dev),
            _dev(b, "b", (B, Lb, desc.n_v), desc.act, dev),
            _dev(lens, "lens", (B,), torch.int32, dev),
            _dev(conv_tail, "conv_tail", (B, desc.kc, desc.conv_dim), desc.act, dev),
            _dev(state, "state", (B, desc.n_v, desc.d_k, desc.d_v), torch.float32, dev),
            _dev(out, "out", (B, Lb, nvd), desc.out, dev))
    wsp = _dev(ws, "ws", None, torch.uint8, dev)
    _check("gdn_prefill_chunk", lib.gdn_prefill_chunk(ctypes.byref(desc.c()), ctypes.byref(cw), *args, B, Lb, wsp,
                                                      ws.numel(), _stream()))
    return out


def decode_step(desc: GdnDesc, w: GdnWeights, mixed, z, a, b, slot, conv_tail_pool, state_pool, out=None,
                check_slots: bool = False):
    """One token per sequence; pool rows slot[b] (or b when slot is None) updated in place. Returns out."""
    lib = load_library()
    B = mixed.shape[0]
    dev = mixed.device
    nvd = desc.n_v * desc.d_v
    npool = state_pool.shape[0]
    if out is None:
        out = torch.empty(B, nvd, dtype=desc.out, device=dev)
    if slot is not None and check_slots:
        _check_index(slot, "slot", npool, True)
    if slot is None and B > npool:
        raise ValueError("decode_step: more sequences than pool rows")
    cw = _weights(desc, w, dev)
    args = (_dev(mixed, "mixed", (B, desc.conv_dim), desc.act, dev),
            _dev(z, "z", (B, nvd), desc.act, dev),
            _dev(a, "a", (B, desc.n_v), desc.act, dev),
            _dev(b, "b", (B, desc.n_v), desc.act, dev),
            _opt(slot, "slot", (B,), torch.int32, dev),
            _dev(conv_tail_pool, "conv_tail_pool", (npool, desc.kc, desc.conv_dim), desc.act, dev),
            _dev(state_pool, "state_pool", (npool, desc.n_v, desc.d_k, desc.d_v), torch.float32, dev),
            _dev(out, "out", (B, nvd), desc.out, dev))
    _check("gdn_decode_step", lib.gdn_decode_step(ctypes.byref(desc.c()), ctypes.byref(cw), *args, B, _stream()))
    return out


def verify_with_checkpoints(desc: GdnDesc, w: GdnWeights, mixed, z, a, b, slot, conv_tail_pool, state_pool,
                            ckpt_state=None, ckpt_tail=None, out=None, check_slots: bool = False):
    """T tokens per sequence, one at a time, from pool rows slot[b] (unchanged). Returns
    (ckpt_state [B,T,n_v,d_k,d_v], ckpt_tail [B,T,Kc,C_ch], out [B,T,n_v*d_v])."""
    lib = load_library()
    B, T, _ = mixed.shape
    dev = mixed.device
    nvd = desc.n_v * desc.d_v
    npool = state_pool.shape[0]
    if ckpt_state is None:
        ckpt_state = torch.empty(B, T, desc.n_v, desc.d_k, desc.d_v, dtype=torch.float32, device=dev)
    if ckpt_tail is None:
        ckpt_tail = torch.empty(B, T, desc.kc, desc.conv_dim, dtype=desc.act, device=dev)
    if out is None:
        out = torch.empty(B, T, nvd, dtype=desc.out, device=dev)
    if slot is not None and check_slots:
        _check_index(slot, "slot", npool, False)
    cw = _weights(desc, w, dev)
    args = (_dev(mixed, "mixed", (B, T, desc.conv_dim), desc.act, dev),
            _dev(z, "z", (B, T, nvd), desc.act, dev),
            _dev(a, "a", (B, T, desc.n_v), desc.act, dev),
            _dev(b, "b", (B, T, desc.n_v), desc.act, dev))
    rest = (_opt(slot, "slot", (B,), torch.int32, dev),
            _dev(conv_tail_pool, "conv_tail_pool", (npool, desc.kc, desc.conv_dim), desc.act, dev),
            _dev(state_pool, "state_pool", (npool, desc.n_v, desc.d_k, desc.d_v), torch.float32, dev),
            _dev(ckpt_state, "ckpt_state", (B, T, desc.n_v, desc.d_k, desc.d_v), torch.float32, dev),
            _dev(ckpt_tail, "ckpt_tail", (B, T, desc.kc, desc.conv_dim), desc.act, dev),
            _dev(out, "out", (B, T, nvd), desc.out, dev))
    _check("gdn_verify_with_checkpoints",
           lib.gdn_verify_with_checkpoints(ctypes.byref(desc.c()), ctypes.byref(cw), *args, T, *rest, B, _stream()))
    return ckpt_state, ckpt_tail, out


def verify_paths(desc: GdnDesc, w: GdnWeights, mixed, z, a, b, slot, conv_tail_pool, state_pool,
                 ckpt_state=None, ckpt_tail=None, out=None, check_slots: bool = False):
    """P candidate paths of T tokens per sequence (mixed [B,P,T,C_ch]), every path of sequence b from pool
    row slot[b] (unchanged). Returns (ckpt_state [B,P,T,n_v,d_k,d_v], ckpt_tail [B,P,T,Kc,C_ch],
    out [B,P,T,n_v*d_v])."""
    lib = load_library()
    B, P, T, _ = mixed.shape
    dev = mixed.device
    nvd = desc.n_v * desc.d_v
    npool = state_pool.shape[0]
    if ckpt_state is None:
        ckpt_state = torch.empty(B, P, T, desc.n_v, desc.d_k, desc.d_v, dtype=torch.float32, device=dev)
    if ckpt_tail is None:
        ckpt_tail = torch.empty(B, P, T, desc.kc, desc.conv_dim, dtype=desc.act, device=dev)
    if out is None:
        out = torch.empty(B, P, T, nvd, dtype=desc.out, device=dev)
    if slot is not None and check_slots:
        _check_index(slot, "slot", npool, False)
    cw = _weights(desc, w, dev)
    args = (_dev(mixed, "mixed", (B, P, T, desc.conv_dim), desc.act, dev),
            _dev(z, "z", (B, P, T, nvd), desc.act, dev),
            _dev(a, "a", (B, P, T, desc.n_v), desc.act, dev),
            _dev(b, "b", (B, P, T, desc.n_v), desc.act, dev))
    rest = (_opt(slot, "slot", (B,), torch.int32, dev),
            _dev(conv_tail_pool, "conv_tail_pool", (npool, desc.kc, desc.conv_dim), desc.act, dev),
            _dev(state_pool, "state_pool", (npool, desc.n_v, desc.d_k, desc.d_v), torch.float32, dev),
            _dev(ckpt_state, "ckpt_state", (B, P, T, desc.n_v, desc.d_k, desc.d_v), torch.float32, dev),
            _dev(ckpt_tail, "ckpt_tail", (B, P, T, desc.kc, desc.conv_dim), desc.act, dev),
            _dev(out, "out", (B, P, T, nvd), desc.out, dev))
    _check("gdn_verify_paths",
           lib.gdn_verify_paths(ctypes.byref(desc.c()), ctypes.byref(cw), *args, T, P, *rest, B, _stream()))
    return ckpt_state, ckpt_tail, out


def accept_paths(drafts, preds, want_ckpt_index: bool = True):
    """Winner of P paths per sequence (drafts [B,P,K], preds [B,P,K+1]). Returns (m [B], path [B],
    emitted [B,K+1], n_emitted [B], ckpt_index [B] or None)."""
    lib = load_library()
    B, P, K = drafts.shape
    dev = drafts.device
    m = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty(B, dtype=torch.int32, device=dev)
    em = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    ne = torch.empty(B, dtype=torch.int32, device=dev)
    ci = torch.empty(B, dtype=torch.int32, device=dev) if want_ckpt_index else None
    _check("gdn_accept_paths",
           lib.gdn_accept_paths(_dev(drafts, "drafts", (B, P, K), torch.int32, dev),
                                _dev(preds, "preds", (B, P, K + 1), torch.int32, dev), B, P, K,
                                _dev(m, "m", (B,), torch.int32, dev), _dev(path, "path", (B,), torch.int32, dev),
                                _dev(em, "emitted", None, torch.int32, dev), _dev(ne, "n_emitted", None, torch.int32, dev),
                                _opt(ci, "ckpt_index", (B,), torch.int32, dev), _stream()))
    return m, path, em, ne, ci


def accept(drafts, preds, want_ckpt_index: bool = True):
    """Accepted prefix per sequence. Returns (m [B], emitted [B,K+1], n_emitted [B], ckpt_index [B] or None)."""
    lib = load_library()
    B, K = drafts.shape
    dev = drafts.device
    m = torch.empty(B, dtype=torch.int32, device=dev)
    em = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    ne = torch.empty(B, dtype=torch.int32, device=dev)
    ci = torch.empty(B, dtype=torch.int32, device=dev) if want_ckpt_index else None
    _check("gdn_accept", lib.gdn_accept(_dev(drafts, "drafts", (B, K), torch.int32, dev),
                                        _dev(preds, "preds", (B, K + 1), torch.int32, dev), B, K,
                                        _dev(m, "m", (B,), torch.int32, dev), _dev(em, "emitted", None, torch.int32, dev),
                                        _dev(ne, "n_emitted", None, torch.int32, dev),
                                        _opt(ci, "ckpt_index", (B,), torch.int32, dev), _stream()))
    return m, em, ne, ci


def state_copy(desc: GdnDesc, dst_state, dst_tail, dst_idx, src_state, src_tail, src_idx, n: int):
    """Copy n {state, tail} records src row src_idx[i] (or i) -> dst row dst_idx[i] (or i). dst_state /
    src_state may be None (tails only), dst_tail / src_tail may be None (states only). Pools are viewed as
    [rows, ...] record arrays; any leading shape is flattened."""
    lib = load_library()
    dev = (src_state if src_state is not None else src_tail).device
    rec_s = desc.n_v * desc.d_k * desc.d_v
    rec_t = desc.kc * desc.conv_dim

    def rows(t, per, dtype, name):
        if t is None:
            return None, 0
        if t.numel() % per:
            raise ValueError(f"{name}: {t.numel()} elements is not a whole number of records")
        return _dev(t, name, None, dtype, dev), t.numel() // per

    ds, nds = rows(dst_state, rec_s, torch.float32, "dst_state")
    dt, ndt = rows(dst_tail, rec_t, desc.act, "dst_tail")
    ss, nss = rows(src_state, rec_s, torch.float32, "src_state")
    st, nst = rows(src_tail, rec_t, desc.act, "src_tail")
    nd = min(x for x in (nds, ndt) if x) if (nds or ndt) else 0
    ns = min(x for x in (nss, nst) if x) if (nss or nst) else 0
    if dst_idx is None and n > nd or src_idx is None and n > ns:
        raise ValueError("state_copy: n exceeds the records available")
    di = _opt(dst_idx, "dst_idx", (n,), torch.int32, dev)
    si = _opt(src_idx, "src_idx", (n,), torch.int32, dev)
    _check("gdn_state_copy", lib.gdn_state_copy(ctypes.byref(desc.c()), ds, dt, di, ss, st, si, n, _stream()))


def state_zero(desc: GdnDesc, state, tail, idx=None, n: int = None):
    """Zero n records (idx[i], or i) of a state pool and / or a tail pool (either may be None)."""
    lib = load_library()
    dev = (state if state is not None else tail).device
    if n is None:
        n = (state if state is not None else tail).shape[0] if idx is None else idx.numel()
    sp = _opt(state, "state", None, torch.float32, dev)
    tp = _opt(tail, "tail", None, desc.act, dev)
    _check("gdn_state_zero", lib.gdn_state_zero(ctypes.byref(desc.c()), sp, tp, _opt(idx, "idx", (n,), torch.int32, dev),
                                                n, _stream()))


PCACHE_STATS = ("rows", "hits", "partial", "cold", "plain", "tokens_reused", "tokens_computed", "ckpts_made",
                "evicted", "rows_kept")


class PrefixStateCache:
    """The prefix-state cache of one GDN layer: bookkeeping in libgdn (gdn_pcache_*), the checkpoint pool
    on the GPU, and the row executor (restore or zero, chunked prefill, snapshots), all on the current
    stream in the plan's order."""

    def __init__(self, desc: GdnDesc, slots: int, stride: int = 2048, tail: int = 16, align: int = 64,
                 max_chunk: int = 2048, min_prefix: int = 256, device="cuda"):
        lib = load_library()
        h = ctypes.c_void_p()
        _check("gdn_pcache_create", lib.gdn_pcache_create(slots, stride, tail, align, max_chunk, min_prefix,
                                                          ctypes.byref(h)))
        self._h, self._lib = h, lib
        self.desc, self.max_chunk = desc, max_chunk
        self.state_pool = torch.empty(max(slots, 1), desc.n_v, desc.d_k, desc.d_v, dtype=torch.float32, device=device)
        self.tail_pool = torch.empty(max(slots, 1), desc.kc, desc.conv_dim, dtype=desc.act, device=device)
        self.ws = prefill_workspace(desc, 1, max_chunk, device)
        # 0, 1, 2, ...: one-element views of it serve as chunk lengths and slot indices without a host copy
        self._ramp = torch.arange(max(max_chunk, slots) + 1, dtype=torch.int32, device=device)

    def __del__(self):
        if getattr(self, "_h", None):
            self._lib.gdn_pcache_destroy(self._h)
            self._h = None

    def plan(self, ids, p_state: int) -> dict:
        """Book one row (ids: its tokens) and return its plan."""
        ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        n = len(ids)
        cap = 16
        while True:
            info = (ctypes.c_int32 * 4)()
            bounds = (ctypes.c_int32 * cap)()
            snap = (ctypes.c_int32 * cap)()
            ck = (ctypes.c_int64 * (cap + 1))()
            nb = self._lib.gdn_pcache_row(self._h, ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n, int(p_state),
                                          cap, info, bounds, snap, ck)
            if nb >= 0:
                break
            if cap > n + 16:
                _check("gdn_pcache_row", nb)
            cap *= 4
        return {"restore_slot": info[0], "c0": info[1], "p": info[2], "bounds": list(bounds[:nb]),
                "snap_slot": list(snap[:nb]), "restored": ck[0], "new": list(ck[1:nb + 1]), "n": n}

    def run_row(self, w: GdnWeights, ids, mixed, z, a, b, state, tail, out, p_state: int) -> dict:
        """One row through the layer: mixed [1,n,C_ch], z [1,n,n_v*d_v], a and b [1,n,n_v]; state [1,n_v,d_k,d_v]
        and tail [1,Kc,C_ch] end as the row's final state; out [1,n,n_v*d_v] is written for tokens [c0, n)."""
        d = self.desc
        plan = self.plan(ids, p_state)
        one = lambda v: self._ramp[v:v + 1]
        if plan["restore_slot"] >= 0:
            state_copy(d, state, tail, None, self.state_pool, self.tail_pool, one(plan["restore_slot"]), 1)
        else:
            state_zero(d, state, tail)
        ends = plan["bounds"] + [plan["n"]]
        s = plan["c0"]
        for i, e in enumerate(ends):
            while s < e:
                t = min(e, s + self.max_chunk)
                prefill_chunk(d, w, mixed[:, s:t], z[:, s:t], a[:, s:t], b[:, s:t], one(t - s), tail, state,
                              out[:, s:t], self.ws)
                s = t
            if i < len(plan["bounds"]) and plan["snap_slot"][i] >= 0:
                state_copy(d, self.state_pool, self.tail_pool, one(plan["snap_slot"][i]), state, tail, None, 1)
        return plan

    def stats(self) -> dict:
        v = (ctypes.c_int64 * len(PCACHE_STATS))()
        _check("gdn_pcache_stats", self._lib.gdn_pcache_stats(self._h, v))
        return dict(zip(PCACHE_STATS, list(v)))

    def alive(self) -> list:
        n = self._lib.gdn_pcache_alive(self._h, 0, None)
        v = (ctypes.c_int64 * max(n, 1))()
        self._lib.gdn_pcache_alive(self._h, n, v)
        return list(v[:n])


def state_record_bytes(desc: GdnDesc) -> int:
    return int(load_library().gdn_state_record_bytes(ctypes.byref(desc.c())))


def mfma_probe(blocks: int = 2048, iters: int = 1024) -> float:
    """Run the MFMA throughput probe once and return its achieved dense f16 TFLOP/s (timed by a
    timing session on the current stream)."""
    lib = load_library()
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    timing_begin(4)
    try:
        _check("gdn_mfma_probe", lib.gdn_mfma_probe(_dev(sink, "sink", None, torch.float32), blocks, iters, _stream()))
    finally:
        rec = timing_end(4)
    ms = rec[0][1]
    return blocks * 4 * 2 * iters * 2 * 32 * 32 * 16 / (ms / 1e3) / 1e12


def timing_begin(capacity: int = 1024) -> None:
    """Open a per-launch timing session on this thread (see gdn_timing_begin)."""
    _check("gdn_timing_begin", load_library().gdn_timing_begin(int(capacity)))


def timing_end(cap: int = 1024):
    """Close the session; returns [(kernel name, milliseconds)] in launch order."""
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_float * cap)()
    n = load_library().gdn_timing_end(names, ms, int(cap))
    if n < 0:
        _check("gdn_timing_end", n)
    return [(names[i].decode(), float(ms[i])) for i in range(min(n, cap))]

