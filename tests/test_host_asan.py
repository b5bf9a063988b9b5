"""CPU: the library's host code under AddressSanitizer.

The host side of libthdattn.so (argument and size checks, workspace sizes,
status strings, the padding mask's host checks) is rebuilt with the address
sanitizer (host pass only; the device code is unchanged) and linked
with the other objects of the last build.  A child Python process, with the
sanitizer runtime preloaded, runs every test of test_abi.py against that copy;
any sanitizer report fails the test.  No GPU is touched: those calls all
return before a launch.
"""
import os
import subprocess
import sys

import pytest

from variable_length_packed_amd import _lib
from variable_length_packed_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import inspect, os, sys, tempfile
sys.path.insert(0, os.path.join(sys.argv[1], "tests"))
sys.path.insert(0, sys.argv[1])
import ctypes
from variable_length_packed_amd import _lib
_lib.LIB_PATH = sys.argv[2]
lib = _lib.load()
# the sanitizer runtime is live in this process and the copy is instrumented
assert hasattr(ctypes.CDLL(None), "__asan_report_load8")
import test_abi
n = 0
for name, fn in sorted(vars(test_abi).items()):
    if not name.startswith("test_") or not callable(fn):
        continue
    params = getattr(fn, "pytestmark", [])
    cases = [()]
    for m in params:
        if m.name == "parametrize":
            cases = [c if isinstance(c, tuple) else (c,) for c in m.args[1]]
    sig = inspect.signature(fn).parameters
    for c in cases:
        if "tmp_path" in sig:
            import pathlib
            fn(pathlib.Path(tempfile.mkdtemp()))
        else:
            fn(*c)
        n += 1
print(f"ran {n} host-code cases under the sanitizer", flush=True)
"""


def test_host_code_under_address_sanitizer(tmp_path):
    rt = B.asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc")
    if not os.path.exists(_lib.LIB_PATH):
        B.build_library()
    lib = B.build_host_asan_library(str(tmp_path / "libthdattn_asan.so"))
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:exitcode=23")
    res = subprocess.run([sys.executable, "-c", CHILD, ROOT, lib], env=env, capture_output=True,
                         text=True, timeout=600)
    assert "AddressSanitizer" not in res.stderr, res.stderr[-4000:]
    assert res.returncode == 0, res.stderr[-4000:]
    assert "host-code cases under the sanitizer" in res.stdout
