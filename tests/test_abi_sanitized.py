"""The library's host code (argument checks, workspace layout, capacity arithmetic) under
AddressSanitizer and UndefinedBehaviorSanitizer.

A copy of libmoe.so whose host code is built with both sanitizers (device code is not
instrumented) is driven from a child process with the sanitizer runtime preloaded: shapes
with extreme field values go through every host function and through every entry point
with arguments that fail validation, so no kernel is launched and no GPU is needed.  Any
out-of-bounds access or undefined operation (signed overflow, out-of-range float to int
conversion, ...) aborts the child and fails the test.
"""
import glob
import os
import subprocess
import sys

import pytest

from routing_expert_ffn_router_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import ctypes, itertools, sys
sys.path.insert(0, ROOT)
import routing_expert_ffn_router_amd as moe
lib = moe.load_library(LIB)
big = [-(1 << 62), -1, 0, 1, 2, 3, 8, 64, 65, 128, 1000, 1024, 1025, (1 << 20) + 128,
       (1 << 31) - 1, 1 << 31, 1 << 40, (1 << 62) + 5]
small = [-5, 0, 1, 2, 3, 4, 8, 63, 64, 65, 1 << 30]
offs = (ctypes.c_int64 * len(moe.WS_REGIONS))()
phases = (ctypes.c_int64 * len(moe.PHASES))()
P, W = 1 << 40, 1 << 40  # never dereferenced: every call below fails validation first
n = 0
for T, d, E, k in itertools.product(big[:12] + big[14:], [128, 256, 100, 1 << 20, 1 << 21, -128],
                                    [1, 8, 256, 1024, 1025, 0], [1, 2, 8, 64, 65, 0, -1]):
    for F, cap, dt, fl, ng, mg in ((256, 0, 1, 0, 0, 0), (1 << 20, T, 0, 1, 8, 4),
                                   (128, 1 << 40, 1, 7, 64, 64), (384, -7, 1, 3, 3, 1),
                                   (256, 5, 2, 8, 0, 1)):
        s = moe.shape(T, d, E, k, F, cap, dt, fl, ng, mg)
        b = ctypes.byref(s)
        lib.moe_workspace_size(b); lib.moe_max_rows(b); lib.moe_workspace_layout(b, offs)
        lib.moe_workspace_phases(b, phases)
        assert lib.moe_route(b, P, P, None, None, 0, P, P, None, None) != 0 or T == 0
        lib.moe_dispatch(b, P, P, None, W, P, P, P, P, None, P, P, P, None)
        lib.moe_expert_ffn(b, P, P, P, P, P, None, W, P, None)
        lib.moe_expert_gate_up(b, P, P, P, P, None, W, P, None)
        lib.moe_expert_gate_up_gathered(b, P, P, P, P, P, None, W, P, None)
        lib.moe_expert_down(b, P, P, P, None, W, P, None)
        lib.moe_combine(b, P, P, P, None, None)
        lib.moe_slot_counts(b, P, P, None, None, None)
        lib.moe_layer(b, P, P, None, P, P, P, None, W, P, None, None, None, None, None)
        n += 1
for T, k, E in itertools.product(big, small, small):
    for cf in (-1.0, 0.0, 1e-300, 0.5, 1.0, 1.25, 1e10, 1e300, float("inf"), float("nan")):
        lib.moe_capacity(T, k, E, cf)
for st in range(-10, 3):
    lib.moe_status_string(st)
lib.moe_workspace_size(None); lib.moe_max_rows(None); lib.moe_workspace_layout(None, offs)
lib.moe_workspace_phases(None, phases)
# the host records run for real on host arrays: counts of every size, invalid ones included
import numpy as np
rng = np.random.default_rng(0)
for E in (1, 2, 7, 20, 256, 1024):
    for k in (1, 2, 8):
        n = rng.integers(0, 50, E).astype(np.int32)
        c = np.minimum(n, rng.integers(0, 50, E)).astype(np.int32)
        moe.expert_stats(int(n.sum()) // k, k, n, c)
        moe.expert_stats(0, k, np.zeros(E, np.int32))
        rbs = rng.integers(0, 9, (k, E)).astype(np.int32)
        moe.slot_stats(37, rbs, np.minimum(rbs, 3))
        for ranks in (1, 3, 8):
            moe.placement_load(n, rng.integers(0, ranks, E), ranks, 2)
            moe.placement_load(n, rng.integers(0, ranks, E), ranks, 0)
        bad = n.copy(); bad[-1] = -1
        assert lib.moe_expert_stats(5, k, E, bad.ctypes.data, None, ctypes.byref(moe.ExpertStats())) != 0
        more = n + 1  # kept above routed (a named array: it must outlive the call)
        assert lib.moe_expert_stats(5, k, E, n.ctypes.data, more.ctypes.data, ctypes.byref(moe.ExpertStats())) != 0
        pl = np.full(E, 9, np.int32)
        out = np.zeros(16, np.int64); mtm = np.zeros(2)
        assert lib.moe_placement_load(E, n.ctypes.data, pl.ctypes.data, 4, 2, out.ctypes.data, out.ctypes.data, mtm.ctypes.data) != 0
print("ok", n)
"""


def _runtime():
    found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return found[0] if found else None


def _fresh(lib):
    if not os.path.exists(lib):
        return False
    t = os.path.getmtime(lib)
    srcs = glob.glob(os.path.join(_build.CSRC, "*")) + [os.path.join(ROOT, "include", "moe.h")]
    return all(os.path.getmtime(f) <= t for f in srcs)


def test_host_code_under_address_and_ub_sanitizers():
    rt = _runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this ROCm install")
    lib = _build.LIB_SANITIZED
    if not _fresh(lib):
        _build.build(sanitize=True)
    code = CHILD.replace("ROOT", repr(ROOT)).replace("LIB", repr(lib))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert r.stdout.split()[0] == "ok"
