"""Build the C ABI's host code for the CPU with AddressSanitizer (test infrastructure).

The library's validation, planning and skip logic (``abi.cpp``) is compiled
with g++ -fsanitize=address and linked with ``launch_recorder.cpp`` in place
of the HIP kernels, so the ABI tests can run it under ASan on a host without
a GPU.  Returns the path of the built library, or None when g++ or its ASan
runtime is not available.
"""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "ring_attention_03_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def asan_runtime() -> str | None:
    """Path of g++'s ASan runtime library (to preload into the interpreter), if any."""
    if not shutil.which("g++"):
        return None
    out = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def build(out_dir: str) -> str | None:
    if asan_runtime() is None:
        return None
    os.makedirs(out_dir, exist_ok=True)
    flags = ["-std=c++17", "-O1", "-g", "-fPIC", "-fsanitize=address", "-fno-omit-frame-pointer",
             "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    objs = []
    for src in (os.path.join(CSRC, "abi.cpp"), os.path.join(HERE, "launch_recorder.cpp")):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        subprocess.run(["g++", *flags, "-c", src, "-o", obj], check=True)
        objs.append(obj)
    lib = os.path.join(out_dir, "libattnring_host_asan.so")
    subprocess.run(["g++", "-shared", "-fsanitize=address", *objs, f"-L{ROCM}/lib", "-lamdhip64",
                    f"-Wl,-rpath,{ROCM}/lib", "-o", lib], check=True)
    return lib
