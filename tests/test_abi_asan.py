"""The C ABI's host code under AddressSanitizer (CPU only).

``tests/asan/build_asan.py`` compiles ``abi.cpp`` with g++ -fsanitize=address
and links it with recording stand-ins for the kernel launches.  The ABI test
suite then runs against that build in a child interpreter with the ASan
runtime preloaded, and a driver makes valid calls (which reach the recorded
launches) as well as invalid ones.  Any ASan report fails the test.
"""

import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, os.path.join(HERE, "asan"))

import build_asan  # noqa: E402

DRIVER = r'''
import ctypes, sys
sys.path.insert(0, {root!r})
from ring_attention_03_amd import _native
lib = _native.load_library()
lib.attn_test_last_forward.argtypes = [ctypes.POINTER(ctypes.c_int)] * 3 + [ctypes.POINTER(ctypes.c_int)]
FAKE = 1 << 32

def problem(**kw):
    base = dict(num_seqs=1, total_q=128, total_k=128, num_q_heads=8, num_kv_heads=1, head_dim=64,
                scale=0.0, causal=1)
    base.update(kw)
    p, keep = _native.AttnProblem(), []
    for key, val in base.items():
        if isinstance(val, list):
            arr = (ctypes.c_int32 * len(val))(*val)
            keep.append(arr)
            setattr(p, key, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)))
        else:
            setattr(p, key, val)
    return p, keep

def last():
    n, m, s = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    off = (ctypes.c_int * 65)()
    cnt = lib.attn_test_last_forward(ctypes.byref(n), ctypes.byref(m), ctypes.byref(s), off)
    return cnt, n.value, m.value, list(off[: s.value + 1])

flag = ctypes.c_int32(-1)
# a visible block launches: 128 rows at 8:1 GQA = 2 row tiles of 64 rows (4 heads x 64 rows per workgroup)
p, keep = problem()
assert lib.attn_ring_step(ctypes.byref(p), 0, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, ctypes.byref(flag), None) == 0
assert flag.value == 1
cnt, units, merge, off = last()
assert (cnt, units, merge, off) == (1, 2, 0, [0, 2]), (cnt, units, merge, off)
# the fused step sets the merge flag
assert lib.attn_ring_step_merge(ctypes.byref(p), 0, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, None, None) == 0
assert last()[:3] == (2, 2, 1)
# varlen: the heaviest sequence is planned first (unit prefix over that order)
p, keep = problem(num_seqs=3, total_q=96, total_k=96, cu_q=[0, 10, 80, 96], cu_k=[0, 10, 80, 96])
assert lib.attn_prefill_causal(ctypes.byref(p), 0, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, None) == 0
assert last()[1:] == (4, 0, [0, 2, 3, 4]), last()
# a fully masked block records nothing
p, keep = problem(q_pos0=[0], k_pos0=[500])
assert lib.attn_ring_step(ctypes.byref(p), 0, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, ctypes.byref(flag), None) == 0
assert flag.value == 0 and last()[0] == 3
# the merge call and the 64-sequence maximum
assert lib.attn_ring_merge(16, 4, 64, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None) == 0 and last()[0] == 4
cu = list(range(0, 65 * 2, 2))
p, keep = problem(num_seqs=64, total_q=128, total_k=128, cu_q=cu, cu_k=cu)
assert lib.attn_ring_step(ctypes.byref(p), 0, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, ctypes.byref(flag), None) == 0
assert last()[1] == 64
print("DRIVER_OK")
'''


@pytest.fixture(scope="module")
def asan_env(tmp_path_factory):
    runtime = build_asan.asan_runtime()
    if runtime is None:
        pytest.skip("g++ with an AddressSanitizer runtime is not available")
    lib = build_asan.build(str(tmp_path_factory.mktemp("asan")))
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               ATTNRING_LIB=lib, PYTHONDONTWRITEBYTECODE="1")
    return env


def _run(cmd, env):
    proc = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = proc.stdout + proc.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    return proc, out


def test_abi_suite_under_asan(asan_env):
    proc, out = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                      os.path.join(HERE, "test_abi.py")], asan_env)
    assert proc.returncode == 0, out[-4000:]
    assert " passed" in out


def test_valid_calls_reach_the_launches_under_asan(asan_env):
    proc, out = _run([sys.executable, "-c", DRIVER.format(root=ROOT)], asan_env)
    assert proc.returncode == 0 and "DRIVER_OK" in out, out[-4000:]
