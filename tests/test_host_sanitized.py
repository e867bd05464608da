"""The host part of the library (page map, block tables, layer split, filter and the
reshard's uniqueness check) built a second time with g++ and the address and
undefined-behaviour sanitizers, and the host C-ABI tests run against it in a child
process (the sanitizer runtime has to be loaded before the interpreter's own
libraries, so it cannot join this process)."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name: str) -> str:
    gxx = shutil.which("g++")
    if not gxx:
        return ""
    r = subprocess.run([gxx, f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


@pytest.mark.timeout(600)
def test_host_tests_under_address_and_ub_sanitizers():
    asan = _runtime("libasan.so")
    if not asan:
        pytest.skip("g++ with libasan is not available")
    from context_paged_kv_amd import build as B

    lib = B.build_host_asan()
    env = dict(os.environ)
    env.update({"DCPKV_LIBRARY": lib, "DCPKV_HOST_ONLY": "1", "LD_PRELOAD": asan,
                # the interpreter's own allocations are not this library's: no leak report
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_capi_host.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=540)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
