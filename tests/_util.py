"""Helpers shared by the GPU tests: seeded inputs on host and device, comparisons."""
from __future__ import annotations

import math
import sys

import numpy as np

import moe_inputs as mi
import routing_expert_ffn_router_amd as moe


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(w):
    import torch

    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def moe_dtype(w) -> int:
    return moe.MOE_BF16 if w.dtype == "bf16" else moe.MOE_F32


def shape_of(w, capacity=None) -> moe.MoeShape:
    C = moe.capacity(w.T, w.k, w.E, w.capacity_factor) if capacity is None else capacity
    return moe.shape(w.T, w.d, w.E, w.k, w.F, C, moe_dtype(w))


def host_inputs(w) -> dict:
    """All tensors of a small workload on the host, widened exactly to float32."""
    out = {n: mi.host_tensor_f32(w, n) for n in ("x", "w_router", "w_gate", "w_up", "w_down")}
    out["b_router"] = mi.router_bias(w)
    return out


def device_inputs(w, device="cuda") -> dict:
    """All tensors of a workload generated on the device (same values as host_inputs)."""
    import torch

    out = {n: mi.device_tensor(w, n, device) for n in ("x", "w_router", "w_gate", "w_up",
                                                       "w_down")}
    b = mi.router_bias(w)
    out["b_router"] = None if b is None else torch.from_numpy(b).to(device)
    return out


def to_device(a: np.ndarray, dtype, device="cuda"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype)


def to_host(t) -> np.ndarray:
    import torch

    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref|, the layer's output tolerance measure."""
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref))) / den


OUT_TOL = 2e-2  # max|GPU - ref| <= 2e-2 * max|ref| for the layer output (bf16 in, fp32 acc)


def logits_tol(L_ref: np.ndarray) -> float:
    """Absolute tolerance for fp32 logits: 1e-4 * max|L| (about 100x the typical fp32
    accumulation error of a d <= 7168 dot product of bf16 values)."""
    return 1e-4 * float(np.max(np.abs(L_ref))) if L_ref.size else 0.0


def near_tie_ok(L_ref: np.ndarray, idx_gpu: np.ndarray, idx_ref: np.ndarray, tol: float):
    """Tokens whose selections differ; each must be explained by logits within `tol`."""
    bad = np.nonzero(np.any(idx_gpu != idx_ref, axis=1))[0]
    unexplained = []
    for t in bad:
        g = set(idx_gpu[t].tolist())
        r = set(idx_ref[t].tolist())
        if g == r:  # same set, different order: adjacent values must be near-equal
            vals = L_ref[t, idx_ref[t]]
            if np.max(np.abs(L_ref[t, idx_gpu[t]] - vals)) > 2 * tol:
                unexplained.append(int(t))
            continue
        # the k-th best logit of the oracle vs every swapped-in expert of the GPU
        kth = L_ref[t, idx_ref[t, -1]]
        for e in g - r:
            if abs(L_ref[t, e] - kth) > 2 * tol:
                unexplained.append(int(t))
                break
    return bad, unexplained
