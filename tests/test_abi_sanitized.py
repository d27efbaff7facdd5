"""The C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer.

``tests/asan/build.sh`` compiles santa_api.cpp for the host alone (g++, no
device code, kernel launchers replaced by stubs) with both sanitizers; the ABI
tests then run in a child process with that library loaded in place of
libsanta.so, so every host check, the workspace layout arithmetic and the
status strings execute under the sanitizers.  CPU only."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import pytest
from stochastic_sparse_decode_amd import santa
santa._LIB_PATH = {lib!r}
santa.library()
maps = open("/proc/self/maps").read()
assert "libasan" in maps and "libsanta_asan.so" in maps, "sanitized library not loaded"
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {abi!r}, "-k", "not no_fallback"]))
"""


def _runtime(name):
    out = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="no AddressSanitizer runtime")
def test_abi_tests_pass_under_asan_and_ubsan(tmp_path):
    lib = subprocess.run([os.path.join(ROOT, "tests", "asan", "build.sh"), str(tmp_path)], capture_output=True,
                         text=True)
    assert lib.returncode == 0, lib.stderr
    path = lib.stdout.strip().splitlines()[-1]
    env = dict(os.environ, LD_PRELOAD=_runtime("libasan.so"), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", SANTA_ABI_SANITIZED="1")
    code = CHILD.format(root=ROOT, lib=path, abi=os.path.join(ROOT, "tests", "test_abi.py"))
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert "passed" in res.stdout
