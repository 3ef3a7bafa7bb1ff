"""The library's host code under AddressSanitizer (CPU, no device): the
host-sanitizer build (build_lib.build_host_asan) runs the CPU ABI tests in a
child process that preloads the compiler's sanitizer runtime.  Any invalid
access, use after free or double free in the codebook solvers, table and
plan construction or argument checks ends that process with a report."""

import os
import subprocess
import sys

import pytest

from conftest import ROOT
from packed_cache_decode_amd import build_lib


def test_host_code_under_address_sanitizer():
    rt = build_lib.asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime next to the compiler")
    objs = [os.path.join(build_lib.BUILD, os.path.splitext(s)[0] + ".o") for s, _ in build_lib.SOURCES]
    if not all(os.path.exists(o) for o in objs):
        build_lib.build()
    lib = build_lib.build_host_asan()
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"), "--tq-lib", lib],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
