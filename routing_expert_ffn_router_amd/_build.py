"""Build libmoe.so (the HIP kernels and their C ABI) in place for gfx950.

    python -m routing_expert_ffn_router_amd._build
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
# hash of the sources and flags libmoe.so was built from, written next to the build objects
STAMP = os.path.join(OBJ, "libmoe.sha256")

SOURCES = ["route.hip", "dispatch.hip", "expert_ffn.hip", "combine.hip", "noalloc.hip",
           "moe_abi.cpp", "stats.cpp"]
# the MFMA-rate calibration for the measurement harness, in a library of its own
CALIB_SOURCES = ["calib.hip"]
CALIB_LIB = os.path.join(PKG, "libmoe_calib.so")

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


def source_hash() -> str:
    """sha256 over the library's compiled sources, the headers they include and the compile
    flags."""
    # flags with the repository's location taken out, so a copy elsewhere hashes the same
    h = hashlib.sha256(" ".join(f.replace(ROOT, "") for f in FLAGS).encode())
    files = ([os.path.join(CSRC, f) for f in SOURCES + CALIB_SOURCES] +
             sorted(glob.glob(os.path.join(CSRC, "*.h"))) +
             [os.path.join(ROOT, "include", h) for h in ("moe.h", "moe_calib.h")])
    for f in files:
        if os.path.isfile(f):
            h.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def built_hash() -> str:
    """The source hash recorded when libmoe.so was last built ("" if unknown)."""
    try:
        with open(STAMP) as fh:
            return fh.read().strip()
    except OSError:
        return ""


def is_current() -> bool:
    """libmoe.so and libmoe_calib.so exist and were built from the sources as they are now."""
    return os.path.exists(LIB) and os.path.exists(CALIB_LIB) and built_hash() == source_hash()


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


def _link(lib: str, objs: list, extra: list) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile and link libmoe.so and libmoe_calib.so (or, with sanitize, the host-sanitized
    copy of libmoe.so in _build/)."""
    os.makedirs(os.path.join(OBJ, "sanitized") if sanitize else OBJ, exist_ok=True)
    srcs = SOURCES if sanitize else SOURCES + CALIB_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), srcs))
    lib = LIB_SANITIZED if sanitize else LIB
    _link(lib, objs[:len(SOURCES)], SANITIZE if sanitize else [])
    if not sanitize:
        _link(CALIB_LIB, objs[len(SOURCES):], [])
        with open(STAMP, "w") as fh:
            fh.write(source_hash() + "\n")
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
