"""The C-ABI layer's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds api.hip with host-side ASan (mx_fp4_weight_amd.build_asan) and runs the CPU checks of
tests/test_abi_cpu.py against that library in a child python with the ASan runtime preloaded:
every NULL / shape / alignment / workspace / tree refusal, and the valid calls that end at the
device check, must pass without a sanitizer report.
"""
import os
import shutil
import subprocess
import sys

import pytest

from tests.conftest import ROOT

pytestmark = pytest.mark.slow


def test_abi_checks_under_host_asan():
    if shutil.which(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")) is None:
        pytest.skip("hipcc not available")
    from mx_fp4_weight_amd import build_asan
    rt = build_asan.asan_runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime found")
    lib = build_asan.build()
    env = dict(os.environ, MXS_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join("tests", "test_abi_cpu.py"), "-k", "not fails_loudly"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert "runtime error" not in out, out[-4000:]  # UndefinedBehaviorSanitizer
    assert r.returncode == 0, out[-4000:]
