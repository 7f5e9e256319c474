"""GPU parity on seeded random layer shapes: the whole layer through moe_layer against the
oracle, across token counts, expert counts, k, capacity, widths, dtypes and the routing
variants together, and on wider layers with long reductions.

The shapes are drawn once from a fixed seed (the list is the same on every run), sized so
that the float64 oracle finishes each in a few seconds.  As in the variant tests, the logits
are compared with the oracle's, then the oracle routes from the GPU's fp32 logits, so the
top-k, every dispatch table and the drop counters must match bit for bit and the output
within the layer tolerance.
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
import routing_expert_ffn_router_amd as moe
from _util import OUT_TOL, device_inputs, host_inputs, log, logits_tol, rel_err, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

PAD, SLOT, SEL = (moe.MOE_FLAG_PAD_TO_CAPACITY, moe.MOE_FLAG_SLOT_MAJOR,
                  moe.MOE_FLAG_BIAS_SELECTION_ONLY)


def _random_cases(n=40, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        E = int(rng.choice([1, 2, 3, 5, 8, 12, 16, 40, 64, 128, 256]))
        k = int(rng.integers(1, min(E, 8) + 1))
        d = int(rng.choice([128, 256, 384, 512]))
        F = int(rng.choice([128, 256, 384, 640, 1024]))
        T = int(rng.integers(1, 1600))
        if T * k * d * F > 3e9:  # keeps the oracle's FFN at a few seconds
            continue
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        cf = None if rng.random() < 0.3 else float(rng.choice([0.5, 0.8, 1.0, 1.25, 2.0]))
        zipf = float(rng.choice([0.0, 0.0, 0.3, 1.1]))
        flags = 0
        if rng.random() < 0.3:
            flags |= SLOT
        if cf is not None and rng.random() < 0.3:
            flags |= PAD  # padded rows: at most E * C = about cf * T * k
        if zipf > 0 and rng.random() < 0.3:
            flags |= SEL
        G = M = 0
        if E >= 8 and E % 4 == 0 and rng.random() < 0.3:
            G, M = 4, 2
            if k > M * (E // G):
                G = M = 0
        name = f"rnd{len(cases)}"
        cases.append((mi.Workload(name, T, d, E, k, F, cf, dtype, zipf), flags, G, M))
    return cases


def _long_k_cases(n=16, seed=20261204):
    """Wider layers with long reductions (d and F up to 4096, so 16-64 k-stages per GEMM
    tile): the prefill tiles' full pipelines, and the tail split of down GEMMs with few
    tiles and F >= 2048.  The weights stay small enough for the float64 oracle."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        E = int(rng.choice([2, 3, 4, 8, 16, 64]))
        k = int(rng.integers(1, min(E, 4) + 1))
        d = int(rng.choice([1024, 2048, 4096]))
        F = int(rng.choice([512, 1024, 2048, 4096]))
        if E * d * F > 6.8e7:  # float64 weight copies in the oracle
            continue
        t_max = int(min(4096, 4e9 / (k * d * F)))
        if t_max < 16:
            continue
        T = int(rng.integers(16, t_max + 1))
        dtype = "f32" if rng.random() < 0.1 else "bf16"
        cf = None if rng.random() < 0.3 else float(rng.choice([1.0, 1.25, 2.0]))
        zipf = float(rng.choice([0.0, 0.0, 1.1]))
        flags = SLOT if rng.random() < 0.2 else 0
        cases.append((mi.Workload(f"longk{len(cases)}", T, d, E, k, F, cf, dtype, zipf),
                      flags, 0, 0))
    return cases


CASES = _random_cases()
LONG_K = _long_k_cases()


@pytest.mark.parametrize("w,flags,G,M", CASES, ids=[c[0].name for c in CASES])
def test_random_layer(w, flags, G, M):
    _check_layer(w, flags, G, M)


@pytest.mark.parametrize("w,flags,G,M", LONG_K, ids=[c[0].name for c in LONG_K])
def test_random_layer_long_k(w, flags, G, M):
    _check_layer(w, flags, G, M)


def _check_layer(w, flags, G, M):
    log(f"random layer {w} flags={flags} groups={G}/{M}")
    h = host_inputs(w)
    C = moe.capacity(w.T, w.k, w.E, w.capacity_factor)
    s = moe.shape(w.T, w.d, w.E, w.k, w.F, C,
                  moe.MOE_BF16 if w.dtype == "bf16" else moe.MOE_F32, flags=flags,
                  n_groups=G, topk_groups=M)
    d_in = device_inputs(w)
    lay = moe.MoELayer(s)
    lay(d_in["x"], d_in["w_router"], d_in["b_router"], d_in["w_gate"], d_in["w_up"],
        d_in["w_down"])
    torch.cuda.synchronize()
    assert lay.status.item() == 0
    sel_only = bool(flags & SEL)
    L_ref = oracle.router_logits(h["x"], h["w_router"], None if sel_only else h["b_router"])
    L_gpu = lay.view("logits").cpu().numpy()
    assert float(np.max(np.abs(L_gpu - L_ref))) <= logits_tol(L_ref)
    res = oracle.moe_layer(h["x"], h["w_router"], h["b_router"], h["w_gate"], h["w_up"],
                           h["w_down"], w.k, C, logits=L_gpu, bias_selection_only=sel_only,
                           n_groups=G or 1, topk_groups=M or None,
                           slot_major=bool(flags & SLOT), pad_to_capacity=bool(flags & PAD))
    assert np.array_equal(lay.view("topk_idx").cpu().numpy(), res["topk_idx"])
    assert np.array_equal(lay.view("dest_row").cpu().numpy(), res["dest_row"])
    assert np.array_equal(lay.view("offsets").cpu().numpy(), res["expert_offsets"])
    assert np.array_equal(lay.routed_counts.cpu().numpy(), res["routed_counts"])
    assert np.array_equal(lay.tokens_per_expert.cpu().numpy(), res["tokens_per_expert"])
    drops = lay.drops.cpu().numpy()
    assert drops[0] == res["drops_total"]
    assert np.array_equal(drops[1:w.k + 1], res["drops_per_slot"])
    assert drops[w.k + 1] == res["fully_dropped_tokens"]
    assert np.max(np.abs(lay.view("topk_w").cpu().numpy() - res["topk_w"])) <= 1e-6
    err = rel_err(to_host(lay.out), res["out"])
    log(f"  out rel err {err:.3e}, drops {int(drops[0])}")
    assert err <= (1e-5 if w.dtype == "f32" else OUT_TOL)
