"""GPU parity of the routing and dispatch variants against the CPU oracle.

Variants (moe_shape.flags, n_groups / topk_groups): pad-to-capacity buffers, slot-major drop
priority, a router bias that shifts the selection only, group-limited top-k, and the per-slot
counts of moe_slot_counts.  Routing tables are compared bit for bit, with the oracle routing
from the same fp32 logits the GPU routed from; outputs within the stated tolerances.
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
import routing_expert_ffn_router_amd as moe
from _util import (OUT_TOL, device_inputs, host_inputs, log, logits_tol, rel_err, to_device,
                   to_host, torch_dtype)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

W = mi.Workload
PAD, SLOT, SEL = (moe.MOE_FLAG_PAD_TO_CAPACITY, moe.MOE_FLAG_SLOT_MAJOR,
                  moe.MOE_FLAG_BIAS_SELECTION_ONLY)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load_library()
    yield
    torch.cuda.synchronize()


def _i32(*shape):
    return torch.empty(shape, dtype=torch.int32, device="cuda")


def _logits(rng, T, E, kind):
    if kind == "normal":
        return (rng.standard_normal((T, E)) * 2).astype(np.float32)
    return rng.choice(np.array([-1.0, -0.0, 0.0, 0.5, 1.0], np.float32), size=(T, E))


def _route(s, L, bias=None):
    T, k = s.T, s.k
    idx, w, status = _i32(T, k), torch.empty((T, k), device="cuda"), _i32(1)
    b = None if bias is None else to_device(bias, torch.float32)
    moe.route(s, None, None, b, to_device(L, torch.float32), idx, w, status, logits_given=True)
    torch.cuda.synchronize()
    assert status.item() == 0
    return idx.cpu().numpy(), w.cpu().numpy()


# ------------------------------------------------------------------- selection-only bias
@pytest.mark.parametrize("T,E,k,kind", [(500, 8, 2, "normal"), (300, 256, 8, "ties"),
                                        (100, 64, 4, "normal"), (77, 1000, 16, "normal")])
def test_route_selection_only_bias(T, E, k, kind):
    log(f"route selection-only bias T={T} E={E} k={k} {kind}")
    rng = np.random.default_rng(T + E + k)
    L = _logits(rng, T, E, kind)
    b = (rng.standard_normal(E) * 0.7).astype(np.float32)
    s = moe.shape(T, 128, E, k, 128, 0, moe.MOE_F32, flags=SEL)
    idx, w = _route(s, L, b)
    ref = oracle.select_topk(oracle.selection_logits(L, b), k)
    assert np.array_equal(idx, ref)
    assert np.max(np.abs(w - oracle.gate_weights(L, ref))) <= 1e-6
    # without the flag the same bias is not applied by the top-k (given logits include it)
    idx0, _ = _route(moe.shape(T, 128, E, k, 128, 0, moe.MOE_F32), L, b)
    assert np.array_equal(idx0, oracle.select_topk(L, k))


def test_router_logits_exclude_selection_only_bias():
    w = W("bf16_e8_zipf_sel", 300, 256, 8, 2, 256, 1.25, "bf16", 1.1)
    h = host_inputs(w)
    dt = torch_dtype(w)
    s = moe.shape(w.T, w.d, w.E, w.k, w.F, 0, moe.MOE_BF16, flags=SEL)
    L = torch.empty((w.T, w.E), dtype=torch.float32, device="cuda")
    idx, gw = _i32(w.T, w.k), torch.empty((w.T, w.k), device="cuda")
    moe.route(s, to_device(h["x"], dt), to_device(h["w_router"], dt),
              to_device(h["b_router"], torch.float32), L, idx, gw)
    torch.cuda.synchronize()
    ref = oracle.router_logits(h["x"], h["w_router"], None)
    L_gpu = L.cpu().numpy()
    assert float(np.max(np.abs(L_gpu - ref))) <= logits_tol(ref)
    # routing from the GPU's own logits is exact
    assert np.array_equal(idx.cpu().numpy(),
                          oracle.select_topk(oracle.selection_logits(L_gpu, h["b_router"]), w.k))


# ------------------------------------------------------------------- group-limited top-k
GROUP_CASES = [(400, 8, 2, 4, 1, "ties"), (400, 8, 2, 2, 1, "normal"),
               (300, 256, 8, 8, 4, "normal"), (300, 256, 8, 8, 4, "ties"),
               (200, 64, 6, 64, 6, "ties"), (100, 1024, 16, 32, 3, "normal"),
               (150, 48, 4, 3, 2, "ties"), (50, 6, 3, 3, 2, "normal"),
               (129, 256, 8, 8, 8, "normal"), (64, 128, 1, 16, 1, "ties")]


@pytest.mark.parametrize("T,E,k,G,M,kind", GROUP_CASES)
def test_route_group_limited(T, E, k, G, M, kind):
    log(f"route grouped T={T} E={E} k={k} groups={G} keep={M} {kind}")
    rng = np.random.default_rng(T * 3 + E + G * 7 + M)
    L = _logits(rng, T, E, kind)
    s = moe.shape(T, 128, E, k, 128, 0, moe.MOE_F32, n_groups=G, topk_groups=M)
    idx, w = _route(s, L)
    ref = oracle.select_topk(L, k, n_groups=G, topk_groups=M)
    assert np.array_equal(idx, ref)
    assert np.max(np.abs(w - oracle.gate_weights(L, ref))) <= 1e-6


def test_route_group_limited_with_selection_bias():
    T, E, k, G, M = 257, 256, 8, 8, 4
    rng = np.random.default_rng(99)
    L = _logits(rng, T, E, "normal")
    b = (rng.standard_normal(E) * 0.5).astype(np.float32)
    s = moe.shape(T, 128, E, k, 128, 0, moe.MOE_F32, flags=SEL, n_groups=G, topk_groups=M)
    idx, w = _route(s, L, b)
    ref = oracle.select_topk(oracle.selection_logits(L, b), k, n_groups=G, topk_groups=M)
    assert np.array_equal(idx, ref)
    assert np.max(np.abs(w - oracle.gate_weights(L, ref))) <= 1e-6


# ------------------------------------------------------------------- dispatch variants
DISPATCH_CASES = [  # T, E, k, C, d, dtype, bias s, flags
    (1000, 8, 2, 250, 256, "bf16", 0.8, SLOT),
    (1000, 8, 2, 250, 256, "bf16", 0.8, PAD),
    (1000, 8, 2, 250, 256, "bf16", 0.8, PAD | SLOT),
    (8192, 256, 8, 256, 128, "bf16", 0.05, SLOT),
    (8192, 256, 8, 256, 128, "bf16", 0.05, PAD),
    (513, 5, 3, 100, 128, "f32", 0.3, SLOT),
    (513, 5, 3, 100, 128, "f32", 0.3, PAD | SLOT),
    (2000, 1024, 64, 50, 128, "bf16", 0.01, SLOT),
    (3, 3, 2, 1, 128, "f32", 0.0, PAD | SLOT),
    (37, 256, 8, 0, 128, "bf16", 0.0, PAD),  # no limit: C = T slots per expert
    (100, 1, 1, 40, 128, "f32", 0.0, PAD),
    # just past the one-block dispatch's 2048 assignments (tiled), and at them (one block)
    (1030, 8, 2, 300, 128, "bf16", 0.3, SLOT),
    (256, 256, 8, 12, 128, "bf16", 0.05, PAD | SLOT),
    (4100, 8, 2, 1100, 128, "bf16", 0.3, SLOT),
    (1024, 256, 8, 40, 128, "bf16", 0.05, PAD | SLOT),
]


def _run_dispatch(s, idx_np, x_np, dt):
    T, E, k, d = s.T, s.E, s.k, s.d
    R = moe.max_rows(s)
    ws = torch.empty(moe.workspace_size(s), dtype=torch.uint8, device="cuda")
    g = dict(routed=_i32(E), kept=_i32(E), offsets=_i32(E + 1), src=_i32(R), dest=_i32(T, k),
             drops=_i32(k + 2), x_perm=torch.full((R, d), 7.0, dtype=dt, device="cuda"),
             slot=torch.full((R,), 7777, dtype=torch.int32, device="cuda"))
    moe.dispatch(s, to_device(idx_np, torch.int32), to_device(x_np, dt), ws, g["routed"],
                 g["kept"], g["offsets"], g["src"], g["dest"], g["drops"], g["x_perm"],
                 src_slot=g["slot"])
    torch.cuda.synchronize()
    return R, g


@pytest.mark.parametrize("T,E,k,C,d,dtype,bias,flags", DISPATCH_CASES)
def test_dispatch_variants_bit_exact(T, E, k, C, d, dtype, bias, flags):
    log(f"dispatch T={T} E={E} k={k} C={C} flags={flags}")
    rng = np.random.default_rng(T + 13 * E + 101 * k + flags)
    L = rng.standard_normal((T, E)).astype(np.float32)
    L += (-bias * np.log(np.arange(1, E + 1))).astype(np.float32)[None, :]
    idx = oracle.select_topk(L, k)
    x = rng.standard_normal((T, d)).astype(np.float32)
    if dtype == "bf16":
        x = mi.bf16_bits_to_f32(mi.bf16_rne_np(x))
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    s = moe.shape(T, d, E, k, 128, C, moe.MOE_BF16 if dtype == "bf16" else moe.MOE_F32,
                  flags=flags)
    R, g = _run_dispatch(s, idx, x, dt)
    ref = oracle.dispatch(idx, E, C, slot_major=bool(flags & SLOT),
                          pad_to_capacity=bool(flags & PAD))
    assert R == (ref["n_rows"] if flags & PAD else min(T * k, E * ref["capacity"]))
    assert np.array_equal(g["routed"].cpu().numpy(), ref["routed_counts"])
    assert np.array_equal(g["kept"].cpu().numpy(), ref["tokens_per_expert"])
    assert np.array_equal(g["offsets"].cpu().numpy(), ref["expert_offsets"])
    assert np.array_equal(g["dest"].cpu().numpy(), ref["dest_row"])
    assert np.array_equal(g["src"].cpu().numpy(), ref["src_token"][:R])
    assert np.array_equal(g["slot"].cpu().numpy(), ref["src_slot"][:R])
    drops = g["drops"].cpu().numpy()
    assert drops[0] == ref["drops_total"]
    assert np.array_equal(drops[1:k + 1], ref["drops_per_slot"])
    assert drops[k + 1] == ref["fully_dropped_tokens"]
    n_rows = R if flags & PAD else ref["n_kept"]
    xp = to_host(g["x_perm"][:n_rows])
    want = oracle.permute(x, ref["src_token"], n_rows)
    assert np.array_equal(xp.view(np.uint32), want.view(np.uint32))  # empty slots are zeros


def test_slot_major_counts_fully_dropped_tokens():
    # capacity 1, every token choosing experts (0, 1) except token 1 choosing (1, 0): in
    # slot-major order the first choices of tokens 0 and 1 take the single slot of experts
    # 0 and 1, so every later token is dropped entirely
    T, E, k = 40, 4, 2
    idx = np.tile(np.array([[0, 1]], np.int32), (T, 1))
    idx[1] = [1, 0]
    s = moe.shape(T, 128, E, k, 128, 1, moe.MOE_F32, flags=SLOT)
    R, g = _run_dispatch(s, idx, np.zeros((T, 128), np.float32), torch.float32)
    ref = oracle.dispatch(idx, E, 1, slot_major=True)
    assert ref["fully_dropped_tokens"] == T - 2
    drops = g["drops"].cpu().numpy()
    assert drops[k + 1] == ref["fully_dropped_tokens"] and drops[0] == ref["drops_total"]
    assert np.array_equal(g["dest"].cpu().numpy(), ref["dest_row"])


# ------------------------------------------------------------------- padded expert FFN
@pytest.mark.parametrize("T,d,E,k,F,C,dtype", [(700, 256, 8, 2, 640, 200, "bf16"),
                                               (600, 256, 4, 2, 384, 320, "f32"),
                                               (37, 512, 256, 8, 384, 0, "bf16")])
def test_expert_ffn_padded(T, d, E, k, F, C, dtype):
    w = W("pad_ffn", T, d, E, k, F, None, dtype)
    log(f"padded expert_ffn {w} C={C}")
    h = host_inputs(w)
    dt = torch_dtype(w)
    s = moe.shape(T, d, E, k, F, C, moe.MOE_BF16 if dtype == "bf16" else moe.MOE_F32,
                  flags=PAD)
    L = oracle.router_logits(h["x"], h["w_router"], None)
    idx = oracle.select_topk(L, k)
    tab = oracle.dispatch(idx, E, C, pad_to_capacity=True)
    R = moe.max_rows(s)
    assert R == tab["n_rows"]
    xp = oracle.permute(h["x"], tab["src_token"], R)
    ws = torch.empty(moe.workspace_size(s), dtype=torch.uint8, device="cuda")
    y = torch.full((R, d), 3.0, dtype=dt, device="cuda")
    moe.expert_ffn(s, to_device(xp, dt), to_device(tab["expert_offsets"].astype(np.int32),
                                                   torch.int32),
                   to_device(h["w_gate"], dt), to_device(h["w_up"], dt),
                   to_device(h["w_down"], dt), ws, y)
    torch.cuda.synchronize()
    ref = oracle.expert_ffn(xp, tab["expert_offsets"], h["w_gate"], h["w_up"], h["w_down"])
    got = to_host(y)
    err = rel_err(got, ref)
    log(f"  rows {R}, rel err {err:.3e}")
    assert err <= (1e-5 if dtype == "f32" else OUT_TOL)
    assert np.all(got[tab["src_token"] < 0] == 0)  # empty slots: silu(0) * 0 = 0


# ------------------------------------------------------------------- whole layer
LAYER_CASES = [
    ("bf16_e8_zipf_drops", PAD, 0, 0),
    ("bf16_e8_zipf_drops", SLOT, 0, 0),
    ("bf16_e8_zipf_drops", SEL, 0, 0),
    ("bf16_e256_k8_drops", PAD | SLOT, 8, 4),
    ("bf16_e256_k8_drops", SEL, 8, 4),
    ("bf16_e256_k8_decode", PAD, 0, 0),
    ("tiny_f32", PAD | SLOT | SEL, 2, 1),
    # C = 560 padded rows per expert: the plan takes the 320-row tile and every expert's
    # last tile holds 240 rows (the gate/up GEMM's 256-row tile, a partly filled 320-row
    # tile in the down GEMM)
    ("bf16_e8_tall_pad", PAD, 0, 0),
]
SMALL = {
    "tiny_f32": mi.WORKLOADS["tiny_f32"],
    "bf16_e8_zipf_drops": W("bf16_e8_zipf_drops", 700, 256, 8, 2, 640, 1.25, "bf16", 1.1),
    "bf16_e256_k8_drops": W("bf16_e256_k8_drops", 512, 256, 256, 8, 256, 1.0, "bf16", 0.05),
    "bf16_e256_k8_decode": W("bf16_e256_k8_decode", 37, 512, 256, 8, 384, None, "bf16"),
    "bf16_e8_tall_pad": W("bf16_e8_tall_pad", 1792, 256, 8, 2, 384, 1.25, "bf16", 1.1),
}


@pytest.mark.parametrize("name,flags,G,M", LAYER_CASES)
def test_layer_variants(name, flags, G, M):
    w = SMALL[name]
    log(f"layer {w} flags={flags} groups={G}/{M}")
    h = host_inputs(w)
    C = moe.capacity(w.T, w.k, w.E, w.capacity_factor)
    s = moe.shape(w.T, w.d, w.E, w.k, w.F, C, moe.MOE_BF16 if w.dtype == "bf16" else
                  moe.MOE_F32, flags=flags, n_groups=G, topk_groups=M)
    d_in = device_inputs(w)
    lay = moe.MoELayer(s)
    lay(d_in["x"], d_in["w_router"], d_in["b_router"], d_in["w_gate"], d_in["w_up"],
        d_in["w_down"])
    torch.cuda.synchronize()
    assert lay.status.item() == 0
    sel_only = bool(flags & SEL)
    # S1 against the oracle's logits (unbiased when the bias is selection-only)
    L_ref = oracle.router_logits(h["x"], h["w_router"], None if sel_only else h["b_router"])
    L_gpu = lay.view("logits").cpu().numpy()
    assert float(np.max(np.abs(L_gpu - L_ref))) <= logits_tol(L_ref)
    # S2-S8 with the oracle routing from the GPU's fp32 logits: tables bit-exact
    res = oracle.moe_layer(h["x"], h["w_router"], h["b_router"], h["w_gate"], h["w_up"],
                           h["w_down"], w.k, C, logits=L_gpu, bias_selection_only=sel_only,
                           n_groups=G, topk_groups=M or None, slot_major=bool(flags & SLOT),
                           pad_to_capacity=bool(flags & PAD))
    assert np.array_equal(lay.view("topk_idx").cpu().numpy(), res["topk_idx"])
    assert np.array_equal(lay.view("dest_row").cpu().numpy(), res["dest_row"])
    assert np.array_equal(lay.view("offsets").cpu().numpy(), res["expert_offsets"])
    assert np.array_equal(lay.tokens_per_expert.cpu().numpy(), res["tokens_per_expert"])
    drops = lay.drops.cpu().numpy()
    assert drops[0] == res["drops_total"] and drops[w.k + 1] == res["fully_dropped_tokens"]
    assert np.max(np.abs(lay.view("topk_w").cpu().numpy() - res["topk_w"])) <= 1e-6
    err = rel_err(to_host(lay.out), res["out"])
    log(f"  out rel err {err:.3e}, drops {int(drops[0])}")
    assert err <= (1e-5 if w.dtype == "f32" else OUT_TOL)


# ------------------------------------------------------------------- observability
@pytest.mark.parametrize("T,E,k,C,flags", [(1000, 8, 2, 250, 0), (8192, 256, 8, 256, SLOT),
                                           (300, 1024, 64, 30, 0), (0, 8, 2, 10, 0)])
def test_slot_counts(T, E, k, C, flags):
    rng = np.random.default_rng(T + E)
    L = (rng.standard_normal((T, E)) - 0.3 * np.log(np.arange(1, E + 1))).astype(np.float32)
    idx = oracle.select_topk(L, k) if T else np.zeros((0, k), np.int32)
    s = moe.shape(T, 128, E, k, 128, C, moe.MOE_F32, flags=flags)
    R, g = _run_dispatch(s, idx, np.zeros((T, 128), np.float32), torch.float32)
    rbs, kbs = _i32(k, E), _i32(k, E)
    moe.slot_counts(s, to_device(idx, torch.int32), g["dest"], rbs, kbs)
    torch.cuda.synchronize()
    if T == 0:
        assert rbs.abs().sum().item() == 0 and kbs.abs().sum().item() == 0
        return
    ref = oracle.dispatch(idx, E, C, slot_major=bool(flags & SLOT))
    rec = oracle.routing_record(idx, ref["dest_row"], E)
    assert rbs.cpu().numpy().tolist() == rec["routed_by_slot"]
    assert kbs.cpu().numpy().tolist() == rec["kept_by_slot"]
    host = moe.routing_record(T, rbs.cpu().numpy(), kbs.cpu().numpy())
    assert host["top_5_percent_expert_share"] == pytest.approx(rec["top_5_percent_expert_share"])
    assert host["drop_share_per_slot"] == pytest.approx(rec["drop_share_per_slot"])
    assert host["slot_max_to_mean"] == pytest.approx(rec["slot_max_to_mean"])


def test_slot_counts_skip_invalid_ids():
    T, E, k = 200, 6, 3
    rng = np.random.default_rng(3)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    inval = rng.random((T, k)) < 0.1
    idx_gpu = np.where(inval, np.where(rng.random((T, k)) < 0.5, -1, E), idx).astype(np.int32)
    dest = np.where(inval, -1, 0).astype(np.int32)
    s = moe.shape(T, 128, E, k, 128, 0, moe.MOE_F32)
    rbs, kbs = _i32(k, E), _i32(k, E)
    moe.slot_counts(s, to_device(idx_gpu, torch.int32), to_device(dest, torch.int32), rbs, kbs)
    torch.cuda.synchronize()
    want = np.zeros((k, E), np.int64)
    for j in range(k):
        np.add.at(want[j], idx[:, j][~inval[:, j]], 1)
    assert np.array_equal(rbs.cpu().numpy(), want)
    assert np.array_equal(kbs.cpu().numpy(), want)
