"""The C ABI's host code under the address and undefined-behaviour
sanitizers: tests/test_boundary.py (argument checks, status codes, exported
symbols; every call is rejected before any launch) runs in a subprocess
against libattn_hostcheck.so -- attn_api.cpp and the no-allocation entry
point compiled with -fsanitize=address,undefined on the host side, with
stub launchers -- and the sanitizer runtime preloaded.  Any report fails
the run (halt on the first error).  CPU only."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_boundary_checks_under_asan_and_ubsan():
    rt = _asan_runtime()
    if rt is None or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc or the clang sanitizer runtime is not installed")
    from exact_attention_tile_amd import build
    lib = build.build_host_check()
    env = dict(os.environ)
    env.update({
        "EXACT_ATTN_LIB": lib,
        "LD_PRELOAD": rt,
        # the interpreter and torch are not instrumented: their leaks and
        # allocator pairing are not this library's
        "ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "PYTHONPATH": ROOT,
    })
    # print which library the binding loaded, then run the boundary tests in
    # the same process
    script = ("import sys, pytest, exact_attention_tile_amd as e\n"
              "print('loaded', e.load_library()._name, flush=True)\n"
              "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', %r]))\n"
              % os.path.join(ROOT, "tests", "test_boundary.py"))
    res = subprocess.run([sys.executable, "-c", script], cwd=ROOT, env=env,
                         stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    tail = res.stdout[-3000:]
    assert "loaded " + lib in res.stdout, tail
    assert "AddressSanitizer" not in res.stdout, tail
    assert "runtime error" not in res.stdout, tail
    assert res.returncode == 0, tail
    assert " passed" in res.stdout, tail
