"""The CPU ABI tests again against librkv_asan.so: the host C++ layer
(argument checks, workspace sizing, error text, the copy-engine staging's
host side) built with AddressSanitizer, in a child process that preloads the
sanitizer runtime.  Any invalid host memory access in those paths aborts the
child with an AddressSanitizer report."""

import os
import subprocess
import sys

import pytest

from sparse_retrieval_kv_amd import build as Bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_tests_under_address_sanitizer():
    if not os.path.exists(Bd.ASAN_LIB):
        pytest.skip("librkv_asan.so not built")
    # the library really is instrumented
    syms = subprocess.run(["nm", "-D", Bd.ASAN_LIB], check=True, stdout=subprocess.PIPE,
                          text=True).stdout
    assert "__asan_init" in syms or "__asan_report" in syms
    env = dict(os.environ, RKV_LIB=Bd.ASAN_LIB, LD_PRELOAD=Bd.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi_host.py", "-q",
                        "-x", "-p", "no:cacheprovider"], cwd=ROOT, env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=900)
    assert "AddressSanitizer" not in r.stdout, r.stdout[-4000:]
    assert r.returncode == 0, r.stdout[-4000:]
