"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library is rebuilt with the sanitizers on its host code only (each -fsanitize is
preceded by -Xarch_host; the gfx950 device code is unchanged), the oracle's C
recurrence with gcc's sanitizers; tests/sanitize_driver.py then drives the planner,
the workspace layout and region queries, the plan cache and every validation path
of the C ABI (fake device pointers: each call fails before a launch), and the oracle,
in a subprocess with the sanitizer runtime preloaded.  Any report fails the test.
Builds are cached under _build/asan by a hash of their sources.
"""
import concurrent.futures
import glob
import hashlib
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_deltanet_chunked_fwd_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]


def _digest(paths, extra):
    h = hashlib.sha256(extra.encode())
    for p in sorted(paths):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def _build_lib():
    srcs = glob.glob(os.path.join(CSRC, "*.hip"))
    deps = srcs + glob.glob(os.path.join(CSRC, "*.h")) + [os.path.join(ROOT, "include", "gdn.h")]
    out = os.path.join(ROOT, "_build", "asan", "gdn_" + _digest(deps, " ".join(HOST_SAN)))
    lib = os.path.join(out, "libgdn_asan.so")
    if os.path.exists(lib):
        return lib
    os.makedirs(out, exist_ok=True)
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC] + HOST_SAN

    def compile_one(src):
        obj = os.path.join(out, os.path.basename(src) + ".o")
        subprocess.run([HIPCC] + flags + ["-c", src, "-o", obj], check=True, capture_output=True)
        return obj
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = lib + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + HOST_SAN + ["-o", tmp] + objs,
                   check=True, capture_output=True)
    os.replace(tmp, lib)
    return lib


def _build_oracle():
    src = os.path.join(ROOT, "oracle", "token_recurrence.c")
    flags = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fopenmp",
             "-fPIC", "-shared", "-std=c99"]
    out = os.path.join(ROOT, "_build", "asan", "oracle_" + _digest([src], " ".join(flags)))
    lib = os.path.join(out, "liboracle_asan.so")
    if not os.path.exists(lib):
        os.makedirs(out, exist_ok=True)
        subprocess.run(["gcc"] + flags + ["-o", lib, src, "-lm"], check=True, capture_output=True)
    return lib


def _run(mode, lib, runtime):
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="3")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize_driver.py"), mode, lib],
                       env=env, capture_output=True, text=True, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "ERROR: AddressSanitizer" not in report and "runtime error:" not in report, report[-4000:]
    return report


def test_abi_host_code_under_asan_ubsan():
    rt = sorted(glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not os.path.exists(HIPCC) or not rt:
        pytest.skip("hipcc or clang's AddressSanitizer runtime not found")
    out = _run("abi", _build_lib(), rt[-1])
    assert "abi ok" in out


def test_oracle_under_asan_ubsan():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("gcc's AddressSanitizer runtime not found")
    out = _run("oracle", _build_oracle(), rt)
    assert "oracle ok" in out
