"""Build ``libattnring.so`` (and the measurement probe ``libattnprobe.so``)
in-tree with hipcc for gfx950.

Usage: ``python -m ring_attention_03_amd.build`` (or ``__graft_entry__.build()``).
Each source compiles to an object in parallel, then each shared library is
linked next to this file.  All device code is built without packed-fp32
instructions.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattnring.so")
SOURCES = ["fwd_bf16.hip", "fwd_f32.hip", "merge.hip", "abi.cpp"]
# matrix-core and vector-ALU rate probes (bench.py --mfma-ceiling, --valu-rates); not part of the attention ABI
PROBE_LIB = os.path.join(PKG, "libattnprobe.so")
PROBE_SOURCES = ["probe_mfma.hip", "probe_valu.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source device flags.  The attention kernel never produces NaNs (its only
# non-finite value is the -inf of masked scores), so it runs with the IEEE mode
# bit off: max/min then need no operand canonicalization, which would otherwise
# double the cost of the row max.
EXTRA = {"fwd_bf16.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"]}


def _compile_cmd(src: str) -> tuple[list[str], str]:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, *COMMON, *DEVICE, *EXTRA.get(src, []), "-x", "hip", "-c", path, "-o", obj]
    else:  # host-only C++ (validation, planning, launches through the HIP runtime)
        cmd = [HIPCC, *COMMON, "-c", path, "-o", obj]
    return cmd, obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs, objs = [], {}
    for src in SOURCES + PROBE_SOURCES:
        cmd, obj = _compile_cmd(src)
        objs[src] = obj
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, proc in procs:
        out, _ = proc.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature; that warning is expected
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if proc.returncode != 0:
            failed.append(src)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    for lib, srcs in ((LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)):
        tmp = lib + ".tmp"
        link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[objs[x] for x in srcs], "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
