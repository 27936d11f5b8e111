"""The library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: the block manager (free queues,
reference counts, prefix-cache hashes, token tables) and the argument
checks and size queries of every entry point, and random serving traces
through the block manager.  A sanitized copy of the
library is built in a temporary directory (host code instrumented, device
code as usual) and the ABI and block-manager suites run against it in a
child process with the ASan runtime preloaded; any report fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_and_block_manager_under_asan_ubsan(tmp_path):
    from paged_kv_cache_51_amd import build
    lib = build.build(force=True, out=str(tmp_path / "libpagedkv.so"), sanitize=True)
    env = dict(os.environ)
    env.update({
        "PKV_LIB": lib,
        "LD_PRELOAD": build.asan_runtime(),
        # python's own small-object allocator hides ctypes buffers from ASan
        "PYTHONMALLOC": "malloc",
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=99",
        "UBSAN_OPTIONS": "print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "tests/test_block_manager.py",
                        "tests/test_serving_trace_host.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
