"""The host library under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU.  host.cpp (validation, planning, plan objects, staging events,
argument checks of every entry point) is rebuilt with both sanitizers on its
host code only (hipcc -Xarch_host -fsanitize=...), linked with the kernel
objects of the ordinary build into a separate library, and
tests/test_host_library.py runs against that library in a child process with
the sanitizer runtime preloaded.  Any report -- an out-of-bounds access, a
use after free, signed overflow, an invalid shift -- fails the child.  No
kernel runs: those tests call only host code."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "paged_kv_cache_plan_amd")
BUILD = os.path.join(PKG, "_build")


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_host_library_under_asan_and_ubsan(tmp_path):
    from paged_kv_cache_plan_amd import _build
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime in /opt/rocm/llvm")
    kernels = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in _build.SOURCES if s != "host.cpp"]
    if not all(os.path.exists(k) for k in kernels):
        _build.build()
    host_o = str(tmp_path / "host_san.o")
    lib = str(tmp_path / "libpkv_san.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-Xarch_host", "-g"]
    cc = subprocess.run([_build._hipcc(), "-x", "hip", *_build.FLAGS, *san, "-c", os.path.join(PKG, "csrc", "host.cpp"),
                         "-o", host_o], capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr[-3000:]
    ld = subprocess.run([_build._hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", host_o, *kernels, "-o", lib],
                        capture_output=True, text=True)
    assert ld.returncode == 0, ld.stderr[-3000:]
    env = dict(os.environ, PKV_LIB_PATH=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86:handle_segv=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=87")
    run = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_host_library.py"),
                          "-q", "-x", "-p", "no:cacheprovider", "-n", "4"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    out = run.stdout[-4000:] + run.stderr[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
    assert run.returncode == 0, out
    assert " passed" in run.stdout, out
