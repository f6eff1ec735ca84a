"""The C ABI's host layer (argument validation, workspace sizing, error
reporting in api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer,
no GPU needed.

api.cpp is compiled again with the sanitizers on its host code only (each
``-fsanitize=`` follows ``-Xarch_host``; device code is built as usual) and
linked with the library's other objects into a separate shared library.  The
CPU ABI tests then run against that library in a child process with the
sanitizer runtime preloaded: every invalid-argument path, the size overflow
guards and the error-message formatting run instrumented, and any report ends
the child with a non-zero status.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from rmsnorm_linear_projection_amd import build_lib  # noqa: E402

OUT = os.path.join(ROOT, "_build", "host_sanitized")
LIB = os.path.join(OUT, "librnl_host_sanitized.so")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.fixture(scope="module")
def sanitized_lib():
    rt = _runtime()
    if rt is None:
        pytest.skip("the clang AddressSanitizer runtime is not installed")
    hipcc = build_lib._hipcc()
    objs = {os.path.basename(s): os.path.join(build_lib.BUILD, os.path.basename(s) + ".o")
            for s in build_lib.sources()}
    if not all(os.path.exists(o) for o in objs.values()):
        build_lib.build()
    os.makedirs(OUT, exist_ok=True)
    api_o = os.path.join(OUT, "api.cpp.o")
    # -O1 -g: the sanitizers' usual build; the flags are the library's own otherwise
    flags = [f for f in build_lib.flags() if f != "-O3"]
    _run([hipcc, *flags, "-O1", "-g", *SAN, "-x", "hip", "-c", os.path.join(build_lib.CSRC, "api.cpp"), "-o", api_o])
    others = [o for name, o in objs.items() if name != "api.cpp"]
    _run([hipcc, f"--offload-arch={build_lib.ARCH}", "-shared", "-fPIC", "-shared-libasan", *SAN[:4],
          api_o, *others, "-o", LIB])
    return LIB, rt


def test_library_is_instrumented(sanitized_lib):
    lib, _ = sanitized_lib
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms


def test_abi_validation_under_sanitizers(sanitized_lib):
    lib, rt = sanitized_lib
    code = ("import sys, pytest\n"
            "import rmsnorm_linear_projection_amd as rnl\n"
            f"rnl.LIB_PATH = {lib!r}\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi_cpu.py']))\n")
    env = dict(os.environ, PYTHONPATH=ROOT, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert " passed" in out
