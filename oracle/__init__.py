"""The Gated DeltaNet layer oracle: plain fp64 CPU code. TEST INFRASTRUCTURE ONLY.

Only tests/, the package's smoke() entry and the benchmark's CPU-baseline leg may import this
package. It wraps `gdn_oracle.c` (token-by-token fp64 recurrence, OpenMP over value heads) through
ctypes; nothing here shares code with the HIP path. Inputs are taken as float arrays holding the
exact values the GPU reads (bf16-representable where the GPU reads bf16) and upcast to fp64.

See gdn_oracle.c for the definition of each function and the passages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, IEEE semantics, OpenMP). GDN_ORACLE_LIBRARY names another build
    of the same source to load instead (the sanitizer build of the CPU tests)."""
    if os.environ.get("GDN_ORACLE_LIBRARY"):
        return os.environ["GDN_ORACLE_LIBRARY"]
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared",
                               "-fPIC", "-std=c99", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Dims(ctypes.Structure):
    _fields_ = [("n_k", ctypes.c_int), ("n_v", ctypes.c_int), ("d_k", ctypes.c_int), ("d_v", ctypes.c_int),
                ("conv_k", ctypes.c_int), ("scale", ctypes.c_double), ("l2_eps", ctypes.c_double),
                ("rms_eps", ctypes.c_double)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        I = ctypes.c_int
        _lib.oracle_conv.argtypes = [I, I, I, I, P, P, P, P]
        _lib.oracle_gates.argtypes = [I, I, I, P, P, P, P, P, P]
        _lib.oracle_delta_rule.argtypes = [ctypes.POINTER(_Dims), I, P, P, P, P, P, P, P, I]
        _lib.oracle_gated_rmsnorm.argtypes = [ctypes.c_long, I, P, P, P, ctypes.c_double, P]
        _lib.oracle_layer_forward.argtypes = [ctypes.POINTER(_Dims), I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, I]
        _lib.oracle_layer_forward.restype = I
        _lib.oracle_verify.argtypes = [ctypes.POINTER(_Dims), I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, I]
        _lib.oracle_verify.restype = I
        _lib.oracle_accept.argtypes = [I, I, P, P, P, P, P]
        _lib.oracle_accept_paths.argtypes = [I, I, I, P, P, P, P, P, P]
    return _lib


def default_threads() -> int:
    n = os.environ.get("OMP_NUM_THREADS")
    if n and n.isdigit():
        return max(1, int(n))
    return max(1, len(os.sched_getaffinity(0)))


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


@dataclass
class Dims:
    n_k: int
    n_v: int
    d_k: int
    d_v: int
    conv_k: int = 4
    scale: float | None = None
    l2_eps: float = 1e-6
    rms_eps: float = 1e-6

    @classmethod
    def of(cls, d) -> "Dims":
        """From any object with the same field names (e.g. gdn_inputs.LayerDims)."""
        return cls(d.n_k, d.n_v, d.d_k, d.d_v, d.conv_k, getattr(d, "scale", None), d.l2_eps, d.rms_eps)

    @property
    def conv_dim(self) -> int:
        return 2 * self.n_k * self.d_k + self.n_v * self.d_v

    def c(self) -> _Dims:
        s = float(self.d_k) ** -0.5 if self.scale is None else float(self.scale)
        return _Dims(self.n_k, self.n_v, self.d_k, self.d_v, self.conv_k, s, self.l2_eps, self.rms_eps)


def conv(w, tail, x, length=None):
    """Causal conv + SiLU over [tail | x] for one sequence. Returns (y [L,C], new tail [Kc,C])."""
    w, x = _f64(w), _f64(x)
    tail = _f64(tail).copy()
    L, C = x.shape
    K = w.shape[1]
    y = np.empty((L, C), dtype=np.float64)
    _load().oracle_conv(C, K, L, L if length is None else int(length), _p(w), _p(tail), _p(x), _p(y))
    return y, tail


def gates(A_log, dt_bias, a, b, length=None):
    """(g, beta) for one sequence; a, b: [L, n_v]."""
    a, b, A_log, dt_bias = _f64(a), _f64(b), _f64(A_log), _f64(dt_bias)
    L, nv = a.shape
    g = np.empty_like(a)
    beta = np.empty_like(a)
    _load().oracle_gates(nv, L, L if length is None else int(length), _p(A_log), _p(dt_bias), _p(a), _p(b),
                         _p(g), _p(beta))
    return g, beta


def delta_rule(dims: Dims, q, k, v, g, beta, H0=None, threads=None):
    """Core recurrence for one sequence: q,k [L,n_k,d_k] raw (L2-normalised inside), v [L,n_v,d_v],
    g, beta [L,n_v], H0 [n_v,d_k,d_v]. Returns (o [L,n_v,d_v], H [n_v,d_k,d_v])."""
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    L = q.shape[0]
    H = np.zeros((dims.n_v, dims.d_k, dims.d_v)) if H0 is None else _f64(H0).copy()
    o = np.empty((L, dims.n_v, dims.d_v))
    cd = dims.c()
    _load().oracle_delta_rule(ctypes.byref(cd), L, _p(q), _p(k), _p(v), _p(g), _p(beta), _p(H), _p(o),
                              threads or default_threads())
    return o, H


def gated_rmsnorm(o, z, w, eps):
    o, z, w = _f64(o), _f64(z), _f64(w)
    dv = o.shape[-1]
    out = np.empty_like(o)
    _load().oracle_gated_rmsnorm(o.size // dv, dv, _p(o), _p(z), _p(w), float(eps), _p(out))
    return out


def layer_forward(dims: Dims, weights, mixed, z, a, b, lens=None, tail=None, H=None, threads=None,
                  want_o=False):
    """Whole layer for B sequences. weights: object with conv_w, A_log, dt_bias, norm_w.
    mixed [B,L,C], z [B,L,n_v*d_v], a/b [B,L,n_v]. Returns dict(out, tail, H[, o])."""
    mixed, z, a, b = _f64(mixed), _f64(z), _f64(a), _f64(b)
    B, L, C = mixed.shape
    assert C == dims.conv_dim
    Kc = dims.conv_k - 1
    lens = _i32(np.full(B, L) if lens is None else lens)
    tail = np.zeros((B, Kc, C)) if tail is None else _f64(tail).copy()
    H = np.zeros((B, dims.n_v, dims.d_k, dims.d_v)) if H is None else _f64(H).copy()
    out = np.empty((B, L, dims.n_v * dims.d_v))
    o = np.empty_like(out) if want_o else None
    cw, al, dt, nw = (_f64(weights.conv_w), _f64(weights.A_log), _f64(weights.dt_bias), _f64(weights.norm_w))
    cd = dims.c()
    rc = _load().oracle_layer_forward(ctypes.byref(cd), B, L, _p(lens), _p(cw), _p(al), _p(dt), _p(nw),
                                      _p(mixed), _p(z), _p(a), _p(b), _p(tail), _p(H), _p(out),
                                      _p(o) if want_o else None, threads or default_threads())
    if rc:
        raise ValueError("oracle_layer_forward rejected its arguments")
    res = {"out": out, "tail": tail, "H": H}
    if want_o:
        res["o"] = o
    return res


def verify(dims: Dims, weights, mixed, z, a, b, tail0, H0, threads=None):
    """T tokens per sequence one at a time from (tail0, H0) (not modified). mixed [B,T,C].
    Returns dict(ckpt_H [B,T,n_v,d_k,d_v], ckpt_tail [B,T,Kc,C], out [B,T,n_v*d_v])."""
    mixed, z, a, b = _f64(mixed), _f64(z), _f64(a), _f64(b)
    B, T, C = mixed.shape
    Kc = dims.conv_k - 1
    tail0, H0 = _f64(tail0), _f64(H0)
    ckH = np.empty((B, T, dims.n_v, dims.d_k, dims.d_v))
    ckT = np.empty((B, T, Kc, C))
    out = np.empty((B, T, dims.n_v * dims.d_v))
    cw, al, dt, nw = (_f64(weights.conv_w), _f64(weights.A_log), _f64(weights.dt_bias), _f64(weights.norm_w))
    cd = dims.c()
    rc = _load().oracle_verify(ctypes.byref(cd), B, T, _p(cw), _p(al), _p(dt), _p(nw), _p(mixed), _p(z), _p(a),
                               _p(b), _p(tail0), _p(H0), _p(ckH), _p(ckT), _p(out), threads or default_threads())
    if rc:
        raise ValueError("oracle_verify rejected its arguments")
    return {"ckpt_H": ckH, "ckpt_tail": ckT, "out": out}


def accept(drafts, preds):
    """drafts [B,K], preds [B,K+1] int. Returns (m [B], emitted [B,K+1], n_emitted [B])."""
    drafts, preds = _i32(drafts), _i32(preds)
    B, K = drafts.shape
    assert preds.shape == (B, K + 1)
    m = np.empty(B, np.int32)
    em = np.empty((B, K + 1), np.int32)
    ne = np.empty(B, np.int32)
    _load().oracle_accept(B, K, _p(drafts), _p(preds), _p(m), _p(em), _p(ne))
    return m, em, ne


def verify_paths(dims: Dims, weights, mixed, z, a, b, tail0, H0, threads=None):
    """P candidate paths per sequence, each T tokens from the sequence's (tail0, H0) (mtp/generate.py
    page, tree_verify_step: the cache is tiled into one row per path and every row runs as an ordinary
    sequence). mixed [B,P,T,C], z [B,P,T,n_v*d_v], a and b [B,P,T,n_v]; tail0 [B,Kc,C], H0 [B,n_v,d_k,d_v].
    Returns dict(ckpt_H [B,P,T,n_v,d_k,d_v], ckpt_tail [B,P,T,Kc,C], out [B,P,T,n_v*d_v])."""
    mixed, z, a, b = _f64(mixed), _f64(z), _f64(a), _f64(b)
    B, P, T = mixed.shape[:3]
    flat = lambda x: x.reshape((B * P,) + x.shape[2:])
    rows = lambda x: np.repeat(_f64(x), P, axis=0)  # row b*P + p starts from sequence b's state
    r = verify(dims, weights, flat(mixed), flat(z), flat(a), flat(b), rows(tail0), rows(H0), threads)
    return {k: v.reshape((B, P) + v.shape[1:]) for k, v in r.items()}


def accept_paths(drafts, preds):
    """drafts [B,P,K], preds [B,P,K+1] int. Returns (m [B], path [B], emitted [B,K+1], n_emitted [B]):
    the first path with the longest accepted prefix, and its emitted tokens."""
    drafts, preds = _i32(drafts), _i32(preds)
    B, P, K = drafts.shape
    assert preds.shape == (B, P, K + 1)
    m = np.empty(B, np.int32)
    path = np.empty(B, np.int32)
    em = np.empty((B, K + 1), np.int32)
    ne = np.empty(B, np.int32)
    _load().oracle_accept_paths(B, P, K, _p(drafts), _p(preds), _p(m), _p(path), _p(em), _p(ne))
    return m, path, em, ne


def state_copy(dst_state, dst_tail, dst_idx, src_state, src_tail, src_idx, n):
    """The fixed-size state record copy (uni_engine.py page, copy_cache_: the records of a sequence's
    recurrent state move between pools with the pools' addresses kept): for i < n, record src_idx[i]
    (or i) of each source pool is written to record dst_idx[i] (or i) of the matching destination pool,
    as it is, bit for bit. Either pair of pools may be None; pools are arrays [rows, ...] updated in
    place. Destination rows must be distinct."""
    si = np.arange(n) if src_idx is None else np.asarray(src_idx, np.int64)[:n]
    di = np.arange(n) if dst_idx is None else np.asarray(dst_idx, np.int64)[:n]
    if len(np.unique(di)) != len(di):
        raise ValueError("state_copy: destination rows must be distinct")
    for dst, src in ((dst_state, src_state), (dst_tail, src_tail)):
        if dst is not None and src is not None:
            dst[di] = src[si]
