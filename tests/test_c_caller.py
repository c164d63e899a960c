"""The C ABI from plain C: tests/c_caller.c, built with gcc -std=c99 -pedantic against include/gdn.h alone and
linked to libgdn.so, makes the host-side calls (version, record and workspace sizes, argument errors, the
prefix-state cache planner) and prints the results, which are checked here. No device work."""
import os
import shutil
import subprocess

import pytest

import gated_delta_rule_44_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_plain_c_caller(tmp_path):
    lib = os.path.abspath(gdn.LIB_PATH)
    if not os.path.exists(lib):
        pytest.skip("libgdn.so is not built")
    exe = str(tmp_path / "c_caller")
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_caller.c"),
                           lib, f"-Wl,-rpath,{os.path.dirname(lib)}",
                           # a sanitized build of the library leaves its runtime to the preloaded one
                           "-Wl,--allow-shlib-undefined", "-o", exe])
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60, check=True).stdout
    got = {line.split(" ", 1)[0]: line.split(" ", 1)[1] for line in out.splitlines()}
    assert "gfx950" in got["version"]
    d = gdn.GdnDesc(n_k=16, n_v=32, d_k=128, d_v=128)
    assert int(got["record"]) == gdn.state_record_bytes(d) == 32 * 128 * 128 * 4 + 3 * 8192 * 2
    assert int(got["workspace"]) == gdn.prefill_workspace_bytes(d, 1, 4096) > 0
    rc, msg = got["decode_null"].split(" ", 1)
    assert int(rc) == -1 and "NULL" in msg  # GDN_EINVAL
    rc, msg = got["conv_unsupported"].split(" ", 1)
    assert int(rc) == -2 and "d_k=48" in msg  # GDN_EUNSUPPORTED
    assert int(got["workspace_unequal"]) == gdn.prefill_workspace_bytes(gdn.GdnDesc(n_k=2, n_v=4, d_k=64, d_v=128), 2,
                                                                         300) > 0
    assert got["pcache"] == "0 0 0 plain=1"
