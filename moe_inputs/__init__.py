"""Seeded synthetic inputs for the MoE layer workloads.

Test and benchmark infrastructure, shared by the CPU oracle side and the GPU side.  It
holds none of the layer's arithmetic: only workload shapes, the counter-based value
generator (``philox_normal.h``, built for the host into ``libmoe_inputs_host.so`` and for
the device into ``libmoe_inputs_dev.so``) and the router-bias recipe.

Workload shapes follow the layers the pages name: Mixtral 8x7B and DeepSeek-V3 as users of
expert parallelism (aiunderstanding.org, "Expert parallelism for MoE serving", deep-dive
section), Mixtral 8x22B in bf16 (polomodov.tech, MegaScale-Infer slides, slide 5), and
DeepSeek-V3's 8 routed experts of 256 (same slides, slide 18).  The pages fix no input
values, so every tensor is synthetic: x ~ N(0, 1), every weight ~ N(0, 1/d_model),
approximated by the Irwin-Hall sum of eight 16-bit uniforms.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

SEED = 0

# Tensor ids: the second Philox key word, one per tensor of a workload.
TENSOR_IDS = {
    "x": 1,
    "w_router": 2,
    "w_gate": 3,
    "w_up": 4,
    "w_down": 5,
    "logits": 6,
    "y": 7,
}


@dataclass(frozen=True)
class Workload:
    """One MoE layer configuration.

    capacity_factor None means no capacity limit (every routed assignment is kept).
    zipf_s > 0 adds the router bias b[e] = -s * ln(e + 1) (expert 0 hottest).
    segments names consecutive token ranges, for reporting per-segment drops.
    """

    name: str
    T: int
    d: int
    E: int
    k: int
    F: int
    capacity_factor: Optional[float]
    dtype: str  # "f32" or "bf16"
    zipf_s: float = 0.0
    segments: tuple = field(default_factory=tuple)

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", T=64, d=128, E=8, k=2, F=256, capacity_factor=2.0,
                         dtype="f32"),
    "mixtral_8x7b_prefill": Workload("mixtral_8x7b_prefill", T=4096, d=4096, E=8, k=2,
                                     F=14336, capacity_factor=1.25, dtype="bf16"),
    "mixtral_8x22b_zipf": Workload("mixtral_8x22b_zipf", T=2048, d=6144, E=8, k=2, F=16384,
                                   capacity_factor=1.25, dtype="bf16", zipf_s=1.1),
    "dsv3_decode": Workload("dsv3_decode", T=256, d=7168, E=256, k=8, F=2048,
                            capacity_factor=None, dtype="bf16"),
    # zipf_s for the mixed batch was calibrated by tests/golden/calibrate_zipf_mixed.py
    # (bisection on the oracle's routing of these exact inputs) so that routed max/mean
    # over experts is about 1.5.
    "dsv3_mixed": Workload("dsv3_mixed", T=8192, d=7168, E=256, k=8, F=2048,
                           capacity_factor=1.0, dtype="bf16", zipf_s=0.04398,
                           segments=(("prefill", 0, 7936), ("decode", 7936, 8192))),
}

ORDER = ["tiny_f32", "mixtral_8x7b_prefill", "mixtral_8x22b_zipf", "dsv3_decode", "dsv3_mixed"]


def normal_scale(std: float) -> np.float32:
    """fp32 factor mapping the Irwin-Hall integer S to a value of standard deviation std."""
    sigma_s = math.sqrt(8.0 * (2.0**32 - 1.0) / 12.0)
    return np.float32(std / sigma_s)


def weight_std(w: Workload) -> float:
    return 1.0 / math.sqrt(w.d)


def tensor_std(w: Workload, name: str) -> float:
    return 1.0 if name == "x" else weight_std(w)


def tensor_shape(w: Workload, name: str) -> tuple:
    return {
        "x": (w.T, w.d),
        "w_router": (w.E, w.d),
        "w_gate": (w.E, w.F, w.d),
        "w_up": (w.E, w.F, w.d),
        "w_down": (w.E, w.d, w.F),
    }[name]


def zipf_bias(E: int, s: float) -> np.ndarray:
    """Router bias b[e] = -s * ln(e + 1), rounded once to fp32 (expert 0 hottest)."""
    e = np.arange(E, dtype=np.float64)
    return (-s * np.log(e + 1.0)).astype(np.float32)


def router_bias(w: Workload) -> Optional[np.ndarray]:
    return zipf_bias(w.E, w.zipf_s) if w.zipf_s > 0 else None


# --------------------------------------------------------------------------------------
# numpy implementation of the generator (slow; pins the compiled one in the CPU tests)
# --------------------------------------------------------------------------------------
_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10_np(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32-10 on uint32 arrays (Salmon et al., SC'11), vectorised over counters."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) for c in (c0, c1, c2, c3))
    for _ in range(10):
        p0 = _M0 * c0
        p1 = _M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        n0 = hi1 ^ c1 ^ np.uint64(k0)
        n2 = hi0 ^ c3 ^ np.uint64(k1)
        c0, c1, c2, c3 = n0, lo1, n2, lo0
        k0 = (k0 + _W0) & 0xFFFFFFFF
        k1 = (k1 + _W1) & 0xFFFFFFFF
    return tuple(c.astype(np.uint32) for c in (c0, c1, c2, c3))


def values_np(seed: int, tensor_id: int, start: int, count: int, scale) -> np.ndarray:
    """fp32 values for element indices [start, start + count), numpy implementation."""
    i = np.arange(start, start + count, dtype=np.uint64)
    words = philox4x32_10_np(i & _MASK32, i >> np.uint64(32), np.zeros_like(i),
                             np.zeros_like(i), seed, tensor_id)
    s = np.zeros(count, dtype=np.int64)
    for wd in words:
        wd = wd.astype(np.int64)
        s += (wd & 0xFFFF) + (wd >> 16)
    s -= 262140
    return s.astype(np.float32) * np.float32(scale)


def bf16_rne_np(v: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits (uint16), round to nearest even; finite inputs."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------------------
# compiled generator (host: OpenMP C; device: HIP)
# --------------------------------------------------------------------------------------
_host_lib = None
_dev_lib = None


def _load(name: str):
    path = os.path.join(_HERE, name)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    return ctypes.CDLL(path)


def host_lib():
    global _host_lib
    if _host_lib is None:
        lib = _load("libmoe_inputs_host.so")
        lib.moe_inputs_fill_host.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                             ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                             ctypes.c_float]
        lib.moe_inputs_fill_host.restype = None
        lib.moe_inputs_bf16_to_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64]
        lib.moe_inputs_bf16_to_f32.restype = None
        _host_lib = lib
    return _host_lib


def dev_lib():
    global _dev_lib
    if _dev_lib is None:
        import torch  # noqa: F401  (bind to the HIP runtime torch loaded; see load_library)

        lib = _load("libmoe_inputs_dev.so")
        lib.moe_inputs_fill_device.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                               ctypes.c_uint64, ctypes.c_uint32,
                                               ctypes.c_uint32, ctypes.c_float, ctypes.c_void_p]
        lib.moe_inputs_fill_device.restype = ctypes.c_int
        _dev_lib = lib
    return _dev_lib


def host_values(tensor_id: int, start: int, count: int, std: float, bf16: bool,
                seed: int = SEED) -> np.ndarray:
    """Values of one tensor slice on the host: uint16 bf16 bits if bf16 else float32."""
    out = np.empty(count, dtype=np.uint16 if bf16 else np.float32)
    host_lib().moe_inputs_fill_host(out.ctypes.data, int(bf16), start, count, seed, tensor_id,
                                    float(normal_scale(std)))
    return out


def host_values_f32(tensor_id: int, start: int, count: int, std: float, bf16: bool,
                    seed: int = SEED) -> np.ndarray:
    """Slice values widened to fp32 (exact for bf16)."""
    v = host_values(tensor_id, start, count, std, bf16, seed)
    if not bf16:
        return v
    out = np.empty(count, dtype=np.float32)
    host_lib().moe_inputs_bf16_to_f32(v.ctypes.data, out.ctypes.data, count)
    return out


def host_tensor_f32(w: Workload, name: str, index0: int = 0, rows: Optional[int] = None
                    ) -> np.ndarray:
    """Tensor `name` of workload w (or rows [index0, index0+rows) of its first axis)."""
    shape = tensor_shape(w, name)
    inner = int(np.prod(shape[1:]))
    rows = shape[0] - index0 if rows is None else rows
    v = host_values_f32(TENSOR_IDS[name], index0 * inner, rows * inner, tensor_std(w, name),
                        w.dtype == "bf16")
    return v.reshape((rows,) + tuple(shape[1:]))


def device_fill(tensor, tensor_id: int, std: float, start: int = 0, seed: int = SEED) -> None:
    """Fill a contiguous torch CUDA tensor (float32 or bfloat16) with generator values."""
    import torch

    assert tensor.is_cuda and tensor.is_contiguous()
    bf16 = tensor.dtype == torch.bfloat16
    assert bf16 or tensor.dtype == torch.float32
    stream = torch.cuda.current_stream(tensor.device).cuda_stream
    rc = dev_lib().moe_inputs_fill_device(tensor.data_ptr(), int(bf16), start, tensor.numel(),
                                          seed, tensor_id, float(normal_scale(std)), stream)
    if rc != 0:
        raise RuntimeError(f"moe_inputs_fill_device failed: hip error {rc}")


def device_tensor(w: Workload, name: str, device="cuda"):
    import torch

    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    t = torch.empty(tensor_shape(w, name), dtype=dt, device=device)
    device_fill(t, TENSOR_IDS[name], tensor_std(w, name))
    return t


def build_commands(py_include: Optional[str] = None) -> list:
    """Shell commands that build the two generator libraries in place."""
    h = os.path.join(_HERE, "libmoe_inputs_host.so")
    d = os.path.join(_HERE, "libmoe_inputs_dev.so")
    return [
        ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
         "-o", h, os.path.join(_HERE, "fill_host.c")],
        ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
         "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-o", d, os.path.join(_HERE, "fill_device.hip")],
    ]
