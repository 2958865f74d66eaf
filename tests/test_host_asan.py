"""The host-side ABI tests again, against a build whose C ABI host code (argument checks,
workspace layouts, dispatch: csrc/api.hip) runs under AddressSanitizer.  CPU only: the GPU
code is not instrumented and no kernel is launched.  Any out-of-bounds access or use after free
in the host code fails the run with the sanitizer's report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_clean_under_host_asan():
    b = pytest.importorskip("linear_recurrent_sequence_gla_amd.build")
    try:
        rt = b.asan_runtime()
    except RuntimeError as e:          # no hipcc
        pytest.skip(str(e))
    if rt is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc's clang")
    try:
        lib = b.build_host_asan()
    except RuntimeError as e:
        pytest.skip(f"host-ASan build not possible here: {e}")
    env = dict(os.environ, GLA_AMD_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=97")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout, out[-2000:]
