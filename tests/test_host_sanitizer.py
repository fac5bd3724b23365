"""The C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer.

build(sanitize=True) (run by __graft_entry__.build) links libgla_san.so: the
host-logic source compiled with -fsanitize=address,undefined and
-fno-sanitize-recover=undefined.  This test reruns the ABI and host-logic tests
in a child process against that library, with the sanitizer runtimes
preloaded; any report fails the child (CPU only, no GPU calls)."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_SAN = os.path.join(ROOT, "recurrent_vision_token_amd", "libgla_san.so")


def _runtime(name):
    out = subprocess.run(["gcc", "-print-file-name=" + name], stdout=subprocess.PIPE, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_abi_and_host_logic_under_sanitizers():
    if not os.path.exists(LIB_SAN):
        pytest.skip("libgla_san.so not built (python recurrent_vision_token_amd/build.py --sanitize)")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc sanitizer runtimes not found")
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan + " " + ubsan, GLA_LIBRARY=LIB_SAN,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_host_logic.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    tail = "\n".join(r.stdout.splitlines()[-30:])
    assert r.returncode == 0, tail
    assert "passed" in tail and "ERROR: AddressSanitizer" not in r.stdout, tail
    assert "runtime error" not in r.stdout, tail
