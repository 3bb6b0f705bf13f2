"""The host block pool built with AddressSanitizer and UndefinedBehaviorSanitizer (g++, host
code only) and driven through its C ABI by randomised operation sequences (tests/pool_fuzz.cpp):
invariants after every call, unchanged state after every failed call, no leak after freeing
everything, and no sanitizer report."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_pool_under_address_and_ub_sanitizers():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "pool_fuzz")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
               "-I", os.path.join(ROOT, "include"),
               os.path.join(ROOT, "kv_cache_attention_kvc_amd", "csrc", "kvc_pool.cpp"),
               os.path.join(ROOT, "tests", "pool_fuzz.cpp"), "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ,
                   ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe, "60", "500"], capture_output=True, text=True, env=env,
                           timeout=300)
        assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
        assert "ok" in r.stdout
