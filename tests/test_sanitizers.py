"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The native range allocator (with the library's error buffer) and the C oracle are built
with g++/gcc and the sanitizers into standalone drivers (tests/sanitize/) that run long
seeded call sequences, edge sizes and invalid calls included.  Any out-of-bounds access,
leak or undefined arithmetic aborts the driver.  No GPU code is built here.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "paged_kv_cache_46_amd", "csrc")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]


def build_and_run(tmp_path, compiler, std, sources, includes=()):
    cc = shutil.which(compiler)
    if cc is None:
        pytest.skip(f"{compiler} not available")
    exe = str(tmp_path / "driver")
    cmd = [cc, std, *SAN, *[f"-I{i}" for i in includes], *sources, "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in r.stderr.lower():
        pytest.skip("sanitizer runtime not available")
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.startswith("OK"), (r.stdout[-2000:] + r.stderr[-4000:])


def test_range_allocator_sanitized(tmp_path):
    build_and_run(tmp_path, "g++", "-std=c++17",
                  [os.path.join(HERE, "sanitize", "alloc_driver.cpp"),
                   os.path.join(CSRC, "range_alloc.cpp"), os.path.join(CSRC, "kvw_error.cpp")],
                  includes=(os.path.join(ROOT, "include"), CSRC))


def test_oracle_sanitized(tmp_path):
    build_and_run(tmp_path, "gcc", "-std=c11",
                  [os.path.join(HERE, "sanitize", "oracle_driver.c"),
                   os.path.join(ROOT, "oracle", "oracle.c")])
