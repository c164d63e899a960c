"""Host-side checks of libgdn.so: it loads, exports every entry point include/gdn.h declares, and its
argument checks reject bad calls before any device work (no kernel is launched here)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_44_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = gdn.load_library()
    names = _declared()
    assert "gdn_prefill_chunk" in names and "gdn_decode_step" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/gdn.h but not exported"
    assert set(names) == set(gdn.EXPORTS)


def test_version_string():
    assert "gfx950" in gdn.version()


def _desc(**kw):
    base = dict(n_k=2, n_v=4, d_k=32, d_v=32)
    base.update(kw)
    return gdn.GdnDesc(**base).c()


def test_unsupported_shapes_are_reported():
    lib = gdn.load_library()
    for kw in (dict(d_k=48, d_v=48), dict(conv_k=3), dict(n_v=6, n_k=4), dict(d_k=64, d_v=48), dict(d_k=16, d_v=32)):
        d = _desc(**kw)
        rc = lib.gdn_conv_chunk(ctypes.byref(d), None, None, None, None, None, 1, 1, None)
        assert rc == -2, (kw, rc)
        assert lib.gdn_last_error()
    # every GQA ratio is built (those other than 1, 2, 4 run in groups), and so is every pair of head dims
    # in {32, 64, 128}: the shape passes, the NULL fails
    for kw in (dict(n_k=1, n_v=8), dict(n_k=2, n_v=6), dict(n_k=1, n_v=3), dict(d_k=64, d_v=32),
               dict(d_k=32, d_v=128), dict(d_k=128, d_v=64)):
        d = _desc(**kw)
        assert lib.gdn_conv_chunk(ctypes.byref(d), None, None, None, None, None, 1, 1, None) == -1, kw


def test_null_and_size_errors():
    lib = gdn.load_library()
    d = _desc()
    assert lib.gdn_conv_chunk(ctypes.byref(d), None, None, None, None, None, 1, 1, None) == -1
    assert b"NULL" in lib.gdn_last_error()
    p = ctypes.c_void_p(256)
    assert lib.gdn_conv_chunk(ctypes.byref(d), p, p, p, ctypes.c_void_p(512), ctypes.c_void_p(768), 0, 4, None) == -1
    # the conv's flattened grid: ceil(C/1024) * ceil(Lb/64) * B workgroups must fit in 2^31
    assert lib.gdn_conv_chunk(ctypes.byref(d), p, p, p, ctypes.c_void_p(512), ctypes.c_void_p(768), 1 << 16,
                              1 << 28, None) == -1
    assert b"2^31" in lib.gdn_last_error()
    assert lib.gdn_accept(None, None, 4, 4, None, None, None, None, None) == -1
    assert lib.gdn_accept_paths(p, p, 4, 2, 4, p, None, p, p, None, None) == -1
    assert b"NULL" in lib.gdn_last_error()
    assert lib.gdn_accept_paths(p, p, 4, 0, 4, p, p, p, p, None, None) == -1 and b"P=0" in lib.gdn_last_error()
    assert lib.gdn_state_copy(ctypes.byref(d), None, None, None, None, None, None, 1, None) == -1
    assert lib.gdn_state_copy(ctypes.byref(d), p, None, None, p, None, None, 1, None) == -1  # aliasing
    w = gdn._Weights(256, 512, 768, 1024)
    # workspace too small is caught before any launch
    rc = lib.gdn_prefill_chunk(ctypes.byref(d), ctypes.byref(w), p, p, p, p, p, p, ctypes.c_void_p(4096),
                               ctypes.c_void_p(8192), 1, 64, ctypes.c_void_p(1 << 20), 16, None)
    assert rc == -1 and b"workspace" in lib.gdn_last_error()
    # verify over paths: checkpoints aliasing the pool, P out of range, B*P over the grid limit
    assert lib.gdn_verify_paths(ctypes.byref(d), ctypes.byref(w), p, p, p, p, 5, 2, None, p, p, p,
                                ctypes.c_void_p(4096), p, 1, None) == -1
    assert b"alias" in lib.gdn_last_error()
    q = ctypes.c_void_p(1 << 24)
    assert lib.gdn_verify_paths(ctypes.byref(d), ctypes.byref(w), p, p, p, p, 5, 0, None, p, p, q, q, p, 1, None) == -1
    assert b"P=0" in lib.gdn_last_error()
    assert lib.gdn_verify_paths(ctypes.byref(d), ctypes.byref(w), p, p, p, p, 5, 4, None, p, p, q, q, p, 20000,
                                None) == -1
    assert b"65535" in lib.gdn_last_error()


def test_sizes():
    lib = gdn.load_library()
    d = gdn.GdnDesc(n_k=16, n_v=32, d_k=128, d_v=128)
    assert gdn.state_record_bytes(d) == 32 * 128 * 128 * 4 + 3 * 8192 * 2
    # d = 128, bf16: from 192 (sequence, head) units on, the fused prefill, which needs no workspace
    assert gdn.prefill_workspace_bytes(d, 8, 100) == 0
    assert gdn.prefill_workspace_bytes(d, 8, 8192) == 0
    assert gdn.prefill_workspace_bytes(d, 6, 4096) == 0
    # fewer units take the two-launch path and its chunk records
    assert gdn.prefill_workspace_bytes(d, 5, 4096) > 0
    # fp32 activations at d = 128 take the two-launch path (records of the bf16 operand layout)
    assert gdn.prefill_workspace_bytes(gdn.GdnDesc(n_k=2, n_v=4, d_k=128, d_v=128, act_dtype=gdn.GDN_F32), 1, 64) > 0
    # a workspace sized for the longest call serves every shorter one (sizes never shrink as Lb grows)
    for dd in (d, gdn.GdnDesc(n_k=16, n_v=16, d_k=128, d_v=128), gdn.GdnDesc(n_k=2, n_v=4, d_k=64, d_v=64)):
        for B in (1, 2, 3, 4, 5, 8):
            sizes = [gdn.prefill_workspace_bytes(dd, B, L) for L in (64, 511, 512, 960, 1024, 1025, 2048, 4096, 8192)]
            assert sizes == sorted(sizes), (dd, B, sizes)


def test_sizes_unequal_head_dims():
    """d_k != d_v: the zero-padded copies at D = max(d_k, d_v) plus the square call's own workspace, which
    never shrinks as Lb grows, and more than the square layer of the smaller dim needs."""
    for dk, dv, act_t in ((64, 128, gdn.GDN_BF16), (128, 32, gdn.GDN_BF16), (32, 64, gdn.GDN_F32)):
        d = gdn.GdnDesc(n_k=2, n_v=4, d_k=dk, d_v=dv, act_dtype=act_t)
        dm = gdn.GdnDesc(n_k=2, n_v=4, d_k=max(dk, dv), d_v=max(dk, dv), act_dtype=act_t)
        for B in (1, 3):
            sizes = [gdn.prefill_workspace_bytes(d, B, L) for L in (1, 64, 65, 300, 1024, 2048)]
            assert sizes == sorted(sizes) and sizes[0] > 0, (dk, dv, B, sizes)
            assert all(s % 256 == 0 for s in sizes)
            # the padded inputs alone: B * L * (2 n_k + n_v) * D activation values
            esz = 2 if act_t == gdn.GDN_BF16 else 4
            assert sizes[-1] >= B * 2048 * (2 * 2 + 4) * max(dk, dv) * esz
            assert sizes[-1] >= gdn.prefill_workspace_bytes(dm, B, 2048)


def test_unequal_dims_workspace_checked():
    """A prefill with key and value heads of different dims checks its (larger) workspace before any
    launch: the square layer's size is too small."""
    lib = gdn.load_library()
    d = gdn.GdnDesc(n_k=2, n_v=4, d_k=64, d_v=128).c()
    dsq = gdn.GdnDesc(n_k=2, n_v=4, d_k=64, d_v=64).c()
    need = lib.gdn_prefill_workspace_bytes(ctypes.byref(d), 1, 300)
    small = lib.gdn_prefill_workspace_bytes(ctypes.byref(dsq), 1, 300)
    assert need > small > 0
    p = ctypes.c_void_p(1 << 20)
    w = gdn._Weights(1 << 20, 1 << 20, 1 << 20, 1 << 20)
    rc = lib.gdn_prefill_chunk(ctypes.byref(d), ctypes.byref(w), p, p, p, p, p, p, p, p, 1, 300, p, small, None)
    assert rc == -1 and b"workspace" in lib.gdn_last_error()


def test_sizes_fused_segments(monkeypatch):
    """The fused path forced for few units: segment maps and states where few units run long calls."""
    monkeypatch.setenv("GDN_PREFILL_PATH", "fused")
    d = gdn.GdnDesc(n_k=16, n_v=32, d_k=128, d_v=128)
    assert gdn.prefill_workspace_bytes(d, 8, 8192) == 0          # 256 units: no segments
    assert gdn.prefill_workspace_bytes(d, 1, 256) == 0           # 4 chunks: too short for segments
    S = 5                                                          # 32 units: min(256 / 64 + 1, 64 / 4)
    assert gdn.prefill_workspace_bytes(d, 1, 4096) == 32 * (2 * (S - 1) + S) * 128 * 128 * 4
    for B in (1, 2, 3, 4, 5):
        sizes = [gdn.prefill_workspace_bytes(d, B, L) for L in (64, 511, 512, 960, 1024, 1025, 2048, 4096, 8192)]
        assert sizes == sorted(sizes), (B, sizes)


def test_sizes_two_phase(monkeypatch):
    """The two-launch path (every shape but d = 128 bf16, or all with GDN_PREFILL_PATH=two_phase): chunk
    records, plus the staged o of split heads."""
    monkeypatch.setenv("GDN_PREFILL_PATH", "two_phase")
    d = gdn.GdnDesc(n_k=16, n_v=32, d_k=128, d_v=128)
    n = gdn.prefill_workspace_bytes(d, 8, 100)
    assert n > 0 and n % 256 == 0
    assert gdn.prefill_workspace_bytes(d, 8, 128) == n  # 100 and 128 tokens both take two chunks
    assert gdn.prefill_workspace_bytes(d, 1, 128) > gdn.prefill_workspace_bytes(d, 1, 100) > 0
    for B in (1, 2, 3, 4, 5):
        sizes = [gdn.prefill_workspace_bytes(d, B, L) for L in (64, 960, 1000, 1023, 1024, 1025, 2048)]
        assert sizes == sorted(sizes), (B, sizes)


def test_desc_out_dtype_checked():
    lib = gdn.load_library()
    d = _desc()
    d.out_dtype = 7
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(d), 1, 64) == 0
    p = ctypes.c_void_p(256)
    w = gdn._Weights(256, 256, 256, 256)
    assert lib.gdn_decode_step(ctypes.byref(d), ctypes.byref(w), p, p, p, p, None, p, p, p, 1, None) == -1
    assert b"out_dtype=7" in lib.gdn_last_error()


def test_python_layer_rejects_cpu_tensors():
    import torch
    d = gdn.GdnDesc(n_k=2, n_v=4, d_k=32, d_v=32)
    x = torch.zeros(1, 4, d.conv_dim, dtype=torch.bfloat16)
    with pytest.raises(RuntimeError):
        gdn.conv_chunk(d, torch.zeros(d.conv_dim, 4, dtype=torch.bfloat16), x, torch.ones(1, dtype=torch.int32),
                       torch.zeros(1, 3, d.conv_dim, dtype=torch.bfloat16))


def test_new_entry_points_reject_bad_arguments():
    """State zero, the MFMA probe and the prefix cache check their arguments before any HIP call."""
    lib = gdn.load_library()
    d = _desc()
    assert lib.gdn_state_zero(ctypes.byref(d), None, None, None, 1, None) == -1 and b"nothing" in lib.gdn_last_error()
    p = ctypes.c_void_p(256)
    assert lib.gdn_state_zero(ctypes.byref(d), p, None, None, 0, None) == -1 and b"n=0" in lib.gdn_last_error()
    assert lib.gdn_state_zero(ctypes.byref(d), ctypes.c_void_p(260), None, None, 1, None) == -1
    assert b"aligned" in lib.gdn_last_error()
    assert lib.gdn_mfma_probe(None, 4, 4, None) == -1 and b"gdn_mfma_probe" in lib.gdn_last_error()
    assert lib.gdn_mfma_probe(p, 0, 4, None) == -1
    h = ctypes.c_void_p()
    assert lib.gdn_pcache_create(4, 512, 16, 64, 0, 0, ctypes.byref(h)) == -1  # max_chunk must be positive
    assert lib.gdn_pcache_create(4, 512, 16, 64, 256, 0, None) == -1
    assert lib.gdn_pcache_create(4, 512, 16, 64, 256, 0, ctypes.byref(h)) == 0
    info = (ctypes.c_int32 * 4)()
    assert lib.gdn_pcache_row(h, None, 5, 5, 0, info, None, None, None) == -1   # ids NULL with n > 0
    assert lib.gdn_pcache_row(h, None, 0, 0, 0, info, None, None, None) == 0    # an empty row: plain
    st = (ctypes.c_int64 * len(gdn.PCACHE_STATS))()
    assert lib.gdn_pcache_stats(h, st) == 0 and st[gdn.PCACHE_STATS.index("plain")] == 1
    assert lib.gdn_pcache_stats(None, st) == -1 and lib.gdn_pcache_alive(h, 0, None) == 0
    lib.gdn_pcache_destroy(h)


def test_timing_session_errors():
    """Session misuse is rejected before any HIP call."""
    lib = gdn.load_library()
    assert lib.gdn_timing_begin(0) == -1 and b"capacity" in lib.gdn_last_error()
    assert lib.gdn_timing_end(None, None, 0) == -1 and b"no open session" in lib.gdn_last_error()



def test_missing_library_fails_loudly():
    """Without libgdn.so every call raises (in a fresh process, the loader pointed at a missing file): no
    entry point has a CPU fallback."""
    import subprocess
    import sys
    code = ("import gated_delta_rule_44_amd as g\n"
            "g.load_library.__defaults__ = ('/nonexistent/libgdn.so',)\n"
            "calls = {'prefill_workspace_bytes': lambda: g.prefill_workspace_bytes(g.GdnDesc(2, 4, 128, 128), 1, 64),\n"
            "         'version': g.version, 'accept': lambda: g.accept(None, None)}\n"
            "for name, f in calls.items():\n"
            "    try:\n"
            "        f()\n"
            "        print(name, 'returned')\n"
            "    except RuntimeError as e:\n"
            "        print(name, 'raised', 'is not built' in str(e))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    lines = sorted(r.stdout.split("\n")[:-1])
    assert lines == ["accept raised True", "prefill_workspace_bytes raised True", "version raised True"], r.stdout + r.stderr
