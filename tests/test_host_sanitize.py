"""The library's host-only entry points (decode, prefill and cache-write
argument validation, the planner, the metadata check) under AddressSanitizer
and UndefinedBehaviorSanitizer.

``host_fuzz/fuzz_validate.cpp`` calls them with valid descriptors in which one
to three fields are replaced by edge values (zero, negative, 2^31, 2^62, the
int64 limits, NULL or misaligned data); every call must return a documented
status, and any signed overflow, out-of-bounds read or other undefined
behaviour aborts the run.  The host sources are plain C++, built here with
g++ (no GPU code is involved)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_attention_decode_attn_amd", "csrc")


def test_host_entry_points_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    exe = str(tmp_path / "fuzz_validate")
    build = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             os.path.join(ROOT, "tests", "host_fuzz", "fuzz_validate.cpp"),
             os.path.join(CSRC, "pa_host.cpp"), os.path.join(CSRC, "pa_prefill_host.cpp"), "-o", exe]
    r = subprocess.run(build, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    for seed in (1, 2):
        r = subprocess.run([exe, "200000", str(seed)], capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
        assert "200000 calls, 0 undocumented statuses" in r.stdout
