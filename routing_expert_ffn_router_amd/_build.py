"""Build libmoe.so (the HIP kernels and their C ABI) in place for gfx950.

    python -m routing_expert_ffn_router_amd._build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")

SOURCES = ["route.hip", "dispatch.hip", "expert_ffn.hip", "combine.hip", "moe_abi.cpp"]

HIPCC = os.environ.get("HIPCC", "hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # no packed fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer (device code is not
# instrumented): the library's argument checks, workspace layout and capacity arithmetic run
# under them in a CPU test.  Each sanitizer flag applies to the host compilation only.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-shared-libasan",
            "-Xarch_host", "-fno-omit-frame-pointer"]
LIB_SANITIZED = os.path.join(OBJ, "libmoe_sanitized.so")


def _compile(src: str, sanitize: bool = False) -> str:
    out = os.path.join(OBJ, "sanitized") if sanitize else OBJ
    obj = os.path.join(out, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    extra = SANITIZE if sanitize else []
    cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile and link libmoe.so (or, with sanitize, the host-sanitized copy in _build/)."""
    os.makedirs(os.path.join(OBJ, "sanitized") if sanitize else OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    lib = LIB_SANITIZED if sanitize else LIB
    tmp = lib + ".tmp"
    extra = SANITIZE if sanitize else []
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
