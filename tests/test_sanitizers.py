"""The host layer of libdspark and the CPU oracle under AddressSanitizer and
UndefinedBehaviorSanitizer, without a GPU.

Both are built with the sanitizers on their host code (the library's device
code is compiled as usual; nothing here launches it) into
_build/sanitize/, keyed by a hash of their sources, and the host-side tests
run against them in a child process whose sanitizer runtime is preloaded:
the oracle's pins and checker tests against the sanitized oracle (gcc's
runtime), and the ABI and dispatch tests against the sanitized library
(clang's runtime). Any report fails the child, and so the test.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build", "sanitize")
CSRC = os.path.join(ROOT, "dspark_block_drafter_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"

SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:symbolize=1",
    "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
}


def _digest(paths) -> str:
    h = hashlib.sha256()
    for p in sorted(paths):
        with open(p, "rb") as f:
            h.update(p.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd[:3])} ... failed:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}")
    return r


def _gcc_runtime() -> str:
    return _run(["gcc", "-print-file-name=libasan.so"]).stdout.strip()


def _clang_runtime() -> str:
    return _run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip()


def build_oracle() -> str:
    src = os.path.join(ROOT, "oracle", "oracle.c")
    out = os.path.join(BUILD, f"liboracle_{_digest([src])}.so")
    if not os.path.exists(out):
        os.makedirs(BUILD, exist_ok=True)
        _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
              "-fPIC", "-shared", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=undefined", src, "-o", out + ".tmp", "-lm"])
        os.replace(out + ".tmp", out)
    return out


def build_library() -> str:
    sys.path.insert(0, ROOT)
    from dspark_block_drafter_amd import build as B
    deps = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(ROOT, "include", "dspark.h")]
    out = os.path.join(BUILD, f"libdspark_{_digest(deps)}.so")
    if os.path.exists(out):
        return out
    os.makedirs(BUILD, exist_ok=True)
    # sanitizers on the host side only (each -fsanitize after -Xarch_host)
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [B.HIPCC, f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), *B.SOURCE_FLAGS.get(src, []), *host_san,
               "-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd)
        return obj

    with ThreadPoolExecutor(len(B.SOURCES)) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    # the link names no HIP source
    link = [CLANG, "-shared", "-fPIC", "-fsanitize=address,undefined", *objs,
            "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", out + ".tmp"]
    _run(link)
    os.replace(out + ".tmp", out)
    for o in objs:
        os.remove(o)
    return out


def _child_pytest(tests, env_extra) -> subprocess.CompletedProcess:
    env = dict(os.environ, **SAN_ENV, **env_extra)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(ROOT, "tests", t) for t in tests]]
    return subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)


def _require(tool: str):
    if subprocess.run(["which", tool], capture_output=True).returncode != 0:
        pytest.skip(f"{tool} is not available")


def test_oracle_under_asan_ubsan():
    _require("gcc")
    lib = build_oracle()
    r = _child_pytest(["test_oracle_pins.py", "test_checker_pins.py"],
                      {"DSPARK_ORACLE_LIB": lib, "LD_PRELOAD": _gcc_runtime()})
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in r.stdout


def test_host_library_under_asan_ubsan():
    if not os.path.exists(CLANG):
        pytest.skip("the ROCm clang is not available")
    lib = build_library()
    r = _child_pytest(["test_abi_cpu.py", "test_dispatch_cpu.py"],
                      {"DSPARK_LIBRARY": lib, "LD_PRELOAD": _clang_runtime()})
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in r.stdout
