"""The oracle and the host side of the C ABI built under AddressSanitizer and UBSan (no GPU).

The C oracle and csrc/capi.cpp (linked with host-only stand-ins for the kernel launchers,
tests/sanitizer_stubs.cpp) are compiled with -fsanitize=address,undefined into a temporary
folder; a child Python process with the sanitizer runtimes preloaded then runs every oracle pin
and every host-ABI test against those builds. Any out-of-bounds access, use after free,
signed overflow or other undefined behaviour aborts the child, and the test fails.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]

DRIVER = r"""
import ctypes, inspect, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle, pins
o = oracle.Oracle(oracle._bind(ctypes.CDLL({oracle_so!r})))
for check in pins.ALL_PINS:
    check(o)
from top_sparse_attention_attn_amd import api
api._LIB_PATH = {capi_so!r}
import test_host_abi
n = 0
for name, fn in sorted(vars(test_host_abi).items()):
    if name.startswith("test_") and callable(fn):
        fn(o) if "oracle_impl" in inspect.signature(fn).parameters else fn()
        n += 1
print("sanitized ok", len(pins.ALL_PINS), n)
"""


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="gcc/g++ not installed")
def test_oracle_pins_and_host_abi_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("sanitizer runtimes not installed")
    oracle_so = str(tmp_path / "liboracle_san.so")
    capi_so = str(tmp_path / "libsparse_attn_host_san.so")
    subprocess.run(["gcc", *SAN, "-std=c11", "-shared", "-fPIC", "-o", oracle_so,
                    os.path.join(ROOT, "oracle", "sparse_attn_oracle.c"), "-lm"], check=True)
    subprocess.run(["g++", *SAN, "-std=c++17", "-shared", "-fPIC", "-o", capi_so,
                    os.path.join(ROOT, "top_sparse_attention_attn_amd", "csrc", "capi.cpp"),
                    os.path.join(HERE, "sanitizer_stubs.cpp")], check=True)
    env = dict(os.environ)
    preload = f"{asan} {ubsan}"
    env["LD_PRELOAD"] = preload + (" " + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = DRIVER.format(root=ROOT, tests=HERE, oracle_so=oracle_so, capi_so=capi_so)
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0 and "sanitized ok" in res.stdout, (res.stdout[-2000:] + res.stderr[-4000:])
