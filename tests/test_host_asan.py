"""The library's host code under AddressSanitizer (CPU, no GPU).

The C ABI's host side (argument checks, shape checks, workspace planning, the top-k scratch
sizing, status strings) is compiled with AddressSanitizer on the host compilation only (the
device code is the product's), and the host-ABI checks of tests/test_abi_host.py run against
that build in a child process with the sanitizer's runtime preloaded. Any heap or stack
overrun, use after free or use of an uninitialised stack slot that the sanitizer catches in
those paths fails the test. Leak checking is off: the HIP runtime keeps allocations for the
life of the process.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    r = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.slow
def test_host_abi_checks_clean_under_address_sanitizer(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("the AddressSanitizer runtime of this toolchain was not found")
    sys.path.insert(0, ROOT)
    from sparse_depth_token_amd import build
    lib = build.build(out=str(tmp_path / "libxmod_asan.so"), build_dir=str(tmp_path / "obj"),
                      host_asan=True)
    env = dict(os.environ, LD_PRELOAD=rt, XMOD_TEST_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out, out[-3000:]
    assert r.returncode == 0 and " passed" in out, out[-3000:]
