"""The host pool under AddressSanitizer and UndefinedBehaviorSanitizer: a
randomized driver (tests/native/pool_fuzz.cpp) calls every pool entry point
with random valid calls, checks the pool's invariants after each, checks
that a call failing for lack of space changes nothing, and ends with every
block free.  Built with g++ for the host only (the pool has no device code)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_327_amd", "csrc")


@pytest.fixture(scope="module")
def fuzz_binary(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    out = tmp_path_factory.mktemp("pool_fuzz") / "pool_fuzz"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "native", "pool_fuzz.cpp"), os.path.join(CSRC, "pool.cpp"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return str(out)


@pytest.mark.parametrize("first", [0, 20])
def test_pool_is_clean_under_sanitizers(fuzz_binary, first):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([fuzz_binary, str(first), "20"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "pool_fuzz ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    counts = [int(w) for w in r.stdout.split() if w.isdigit()]
    assert len(counts) == 4 and all(c > 0 for c in counts[1:]), r.stdout   # hits, copies, refusals
