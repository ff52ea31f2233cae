"""The library's host code (argument checks, workspace plans, schedule choice, launchers) under
AddressSanitizer: a copy of libmsa with ASan-built host code runs the host-only ABI tests in a
child process with the sanitizer runtime preloaded. Any invalid host memory access aborts that
child and fails this test. No GPU is touched (the host tests make no compute call)."""
import os
import subprocess
import sys

import pytest

from block_sparse_gqa_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

RUNNER = """
import sys
sys.path.insert(0, {root!r})
from block_sparse_gqa_amd import msa
msa.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", {tests!r}]))
"""


def test_abi_host_tests_under_address_sanitizer():
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc")
    lib = build.build_asan()
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    code = RUNNER.format(root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi_host.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "AddressSanitizer" not in r.stderr
    assert " passed" in r.stdout
