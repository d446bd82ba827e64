"""The host layer of the C ABI (argument validation, cache layout and views,
the schedule, the Hilbert order) under AddressSanitizer and
UndefinedBehaviorSanitizer: a g++ build of api.cpp and order.cpp with failing
launch stubs runs the host ABI tests and the plain-C check in a child process.
CPU only; no device code is built or run."""
import os
import shutil
import subprocess
import sys

import pytest

from tests.sanitize import build_host

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_layer_under_asan_ubsan(tmp_path):
    lib = build_host.build(str(tmp_path))
    runtime = build_host.asan_runtime()
    if runtime is None:
        pytest.skip("no AddressSanitizer runtime for g++")
    env = dict(os.environ, RETTN_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", CUDA_VISIBLE_DEVICES="", HIP_VISIBLE_DEVICES="")
    probe = ("import ctypes; from sparse_attention_diffusion_amd import rettn; "
             "print(rettn.LIB_PATH); ctypes.CDLL(None).__asan_init")
    out = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.strip() == lib, out.stdout + out.stderr
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi_host.py"), os.path.join(ROOT, "tests", "test_c_abi.py")]
    out = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = out.stdout[-3000:] + out.stderr[-3000:]
    assert out.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report
    assert "passed" in out.stdout
