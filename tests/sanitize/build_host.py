"""Host-only build of the C ABI layer under AddressSanitizer and
UndefinedBehaviorSanitizer (test infrastructure).

api.cpp and order.cpp are compiled with g++ (no device code) and linked with
launch_stub.cpp, whose launches all fail, into ``librettn_host_asan.so``.
``tests/test_sanitized_host.py`` runs the host ABI tests against it.
"""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "sparse_attention_diffusion_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]


def rocm():
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def asan_runtime():
    """The g++ AddressSanitizer runtime, to preload into an uninstrumented python."""
    out = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True, check=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def build(out_dir):
    if shutil.which("g++") is None:
        raise RuntimeError("g++ not found")
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "order.cpp"), os.path.join(HERE, "launch_stub.cpp")):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
               "-I", os.path.join(rocm(), "include"), "-I", os.path.join(ROOT, "include")] + SAN + ["-c", src, "-o", obj]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        objs.append(obj)
    lib = os.path.join(out_dir, "librettn_host_asan.so")
    cmd = ["g++", "-shared"] + SAN + objs + ["-L", os.path.join(rocm(), "lib"), "-lamdhip64",
                                             "-Wl,-rpath," + os.path.join(rocm(), "lib"), "-o", lib]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return lib
