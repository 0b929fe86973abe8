"""The library's host code (pool, views, split/merge allocator, budgets,
adjuster) under AddressSanitizer and UndefinedBehaviorSanitizer: a seeded C++
stress driver (tests/cpp/host_stress.cpp) is compiled with g++ together with
the allocator and adjuster sources and run for several seeds. No GPU code is
involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_moe_expert_amd", "csrc")


@pytest.fixture(scope="module")
def stress_bin(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("san") / "host_stress")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "cpp", "host_stress.cpp"), os.path.join(CSRC, "allocator.cpp"),
           os.path.join(CSRC, "adjuster.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_host_code_clean_under_sanitizers(stress_bin, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([stress_bin, str(seed)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "host stress ok" in r.stdout
