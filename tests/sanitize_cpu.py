"""Run the CPU test suite against AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code.

    python tests/sanitize_cpu.py [extra pytest args]

Builds, under _build/san/:
  liboracle_san.so - the oracle (oracle/gdn_oracle.c) with clang, -fsanitize=address,undefined;
  libgdn_san.so    - the library with its host code (the C ABI's argument checks, workspace sizing,
                     the prefix-state cache planner gdn_pcache.cpp) sanitized and its device code
                     built as usual (the sanitizers apply to the host pass only);
then runs `pytest -m "not gpu"` in a child process with both builds selected (GDN_ORACLE_LIBRARY,
GDN_LIBRARY) and the clang sanitizer runtime preloaded into the interpreter. Any sanitizer report
aborts that process and fails the run. CPU only: nothing here touches a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "san")
LLVM = "/opt/rocm/llvm"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
            "-fno-gpu-sanitize", "-shared-libsan", "-g"]


def runtime() -> str:
    libs = glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    if not libs:
        raise RuntimeError("clang's AddressSanitizer runtime was not found under " + LLVM)
    return libs[0]


def build_oracle() -> str:
    lib = os.path.join(OUT, "liboracle_san.so")
    src = os.path.join(ROOT, "oracle", "gdn_oracle.c")
    subprocess.check_call([os.path.join(LLVM, "bin", "clang"), "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared-libsan",
                           "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-std=c99",
                           src, "-o", lib, "-lm", f"-Wl,-rpath,{LLVM}/lib"])
    return lib


def build_library() -> str:
    sys.path.insert(0, ROOT)
    from gated_delta_rule_44_amd import build as b

    def one(src):
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        subprocess.check_call([b.hipcc(), *b.FLAGS, *HOST_SAN, "-c", os.path.join(b.CSRC, src), "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(min(len(b.SOURCES), int(os.environ.get("MAX_JOBS", "8")))) as ex:
        objs = list(ex.map(one, b.SOURCES))
    lib = os.path.join(OUT, "libgdn_san.so")
    subprocess.check_call([b.hipcc(), f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-shared-libsan",
                           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                           *objs, "-o", lib])
    return lib


def main(argv) -> int:
    os.makedirs(OUT, exist_ok=True)
    env = dict(os.environ)
    env.update(GDN_ORACLE_LIBRARY=build_oracle(), GDN_LIBRARY=build_library(), LD_PRELOAD=runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the child must map the sanitizer runtime and both sanitized builds, not the plain ones
    probe = ("import oracle, gated_delta_rule_44_amd as g; oracle._load(); g.load_library(); "
             "m = open('/proc/self/maps').read(); "
             "print(all(x in m for x in ('libclang_rt.asan', 'liboracle_san.so', 'libgdn_san.so')))")
    seen = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True)
    if seen.stdout.strip() != "True":
        print("sanitized builds not loaded:", seen.stdout, seen.stderr[-2000:], file=sys.stderr)
        return 1
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-q", "-x", "-p",
           "no:cacheprovider", *argv]
    return subprocess.call(cmd, cwd=ROOT, env=env)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
