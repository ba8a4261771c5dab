"""The host-side checks of the C ABI (tests/test_abi_host.py) rerun against a
build whose host code carries the address sanitizer: validation, size
queries and request-table construction must not read or write out of
bounds on any of the error and size paths those checks drive.  No GPU is
touched; device code is not instrumented."""
import os
import subprocess
import sys

import pytest

from block_sparse_long_pooling_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_checks_under_address_sanitizer():
    rt = build.asan_runtime()
    if not rt:
        pytest.skip("no shared address-sanitizer runtime in this toolchain")
    lib = build.build_host_asan()
    env = dict(os.environ, FLASHPREFILL_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0")
    probe = ("import block_sparse_long_pooling_amd as fp; fp.lib(); "
             "print(fp.LIB_PATH); print(open('/proc/self/maps').read().count('libclang_rt.asan'))")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    path, mapped = r.stdout.split()[-2:]
    assert path == lib and int(mapped) > 0
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join("tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "AddressSanitizer" not in r.stderr
