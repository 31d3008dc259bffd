"""The host-side ABI checks (tests/test_abi.py) again, against a build of the library
whose host runtime is compiled with AddressSanitizer: argument and state checks,
table copies and the workspace bookkeeping of validate-only contexts must not read or
write out of bounds, use freed memory or free twice."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs the ROCm toolchain to build the library")
def test_abi_checks_under_address_sanitizer():
    from transformer_decode_amd import build as B
    lib = B.build_asan(verbose=False)
    env = dict(os.environ, LD_PRELOAD=B.asan_runtime(), HE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(HERE, "test_abi.py")], env=env, capture_output=True, text=True,
                       timeout=900, cwd=os.path.dirname(HERE))
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
