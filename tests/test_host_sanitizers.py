"""The host allocator (C++) under AddressSanitizer and UndefinedBehavior-
Sanitizer: a randomized driver (tests/native/host_alloc_fuzz.cpp) calls
every allocator entry point with valid and invalid arguments and checks the
reference-count and free-list invariants after every call.  Host code only,
built with g++ (no device code involved)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def fuzz_binary(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("asan") / "host_alloc_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "paged_kv_attention_slot_amd", "csrc", "host_alloc.cpp"),
           os.path.join(ROOT, "tests", "native", "host_alloc_fuzz.cpp"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_allocator_under_sanitizers(fuzz_binary, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([fuzz_binary, str(seed)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    assert r.stdout.strip().endswith("ok")
