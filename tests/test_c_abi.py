"""The C ABI from plain C: tests/c_abi_check.c is compiled with gcc against
include/rettn.h, linked with the built library and run (host-only calls)."""
import os
import shutil
import subprocess

import pytest

from sparse_attention_diffusion_amd import rettn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_is_c_and_host_calls_work(tmp_path):
    exe = tmp_path / "c_abi_check"
    libdir = os.path.dirname(rettn.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", str(exe), rettn.LIB_PATH,
           "-Wl,-rpath," + libdir]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "ok"


@pytest.mark.gpu
def test_c_program_drives_the_gpu_path():
    """tests/c_gpu_check.c (built by __graft_entry__.build()): selector, calibration,
    R1 and R2 sparse steps and the token reorder driven from C with HIP runtime
    memory only; the sparse steps reproduce the calibration output on its own
    inputs and the reorder round-trips bit for bit."""
    exe = os.path.join(ROOT, "tests", "_bin", "c_gpu_check")
    assert os.path.exists(exe), "build() has not been run"
    print("c_gpu_check", flush=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.strip() == "ok"
