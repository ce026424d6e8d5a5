"""The host C++ (allocator, prefix index with LRU eviction, buddy arena)
under AddressSanitizer and UndefinedBehaviorSanitizer: the host test files,
which drive it through the C ABI against the oracle on random operation
sequences, run again in a child interpreter against a sanitized host-only
build.  Any heap error, use after free, overflow or undefined behaviour
aborts the child."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_host_allocator.py", "tests/test_host_prefix.py",
              "tests/test_host_eviction.py", "tests/test_host_buddy.py"]


def test_host_code_under_asan_and_ubsan():
    # The child is started with fork + exec: never from a process that has
    # touched a GPU.
    if torch.cuda.is_initialized():
        pytest.skip("a GPU is initialised in this process; run the host tests alone")
    sys.path.insert(0, os.path.join(ROOT, "paged_kv_cache_166_amd"))
    try:
        import build_host_san as B
    finally:
        sys.path.pop(0)
    lib = B.build()
    env = dict(os.environ)
    env.update(PA_HOST_LIB=lib, LD_PRELOAD=B.runtime_preload(),
               # the interpreter and torch are not instrumented: their own
               # allocations are not tracked for leaks
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               CUDA_VISIBLE_DEVICES="", HIP_VISIBLE_DEVICES="")
    # the child really runs the sanitized build, with the ASan runtime live
    probe = ("import ctypes, paged_kv_cache_166_amd as pa; "
             "print(pa.lib._name); print(hasattr(ctypes.CDLL(None), '__asan_init'))")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split() == [lib, "True"], r.stdout
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           *HOST_TESTS, "tests/test_abi.py::test_sequences_stop_at_int32_max_tokens"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr, tail
    assert "runtime error" not in r.stderr, tail
