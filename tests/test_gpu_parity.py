"""GPU parity: every C-ABI entry point against the CPU oracle on seeded inputs.

Sizes are small enough for the oracle to finish in seconds but span several tiles of every
kernel and end in ragged tails.  Routing tables and the permutation are compared bit for
bit; floating-point outputs within the tolerances stated next to each check.
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
import routing_expert_ffn_router_amd as moe
from _util import (OUT_TOL, device_inputs, host_inputs, log, logits_tol, near_tie_ok, rel_err,
                   shape_of, to_device, to_host, torch_dtype)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

W = mi.Workload
# small layers: (name, T, d, E, k, F, cf, dtype, zipf_s)
SMALL = {
    "tiny_f32": mi.WORKLOADS["tiny_f32"],
    "bf16_e8_big_tiles": W("bf16_e8_big_tiles", 1000, 384, 8, 2, 384, 1.25, "bf16"),
    "bf16_e8_zipf_drops": W("bf16_e8_zipf_drops", 700, 256, 8, 2, 640, 1.25, "bf16", 1.1),
    "bf16_e16_small_tiles": W("bf16_e16_small_tiles", 64, 384, 16, 2, 640, None, "bf16"),
    "bf16_e256_k8_drops": W("bf16_e256_k8_drops", 512, 256, 256, 8, 256, 1.0, "bf16", 0.05),
    "bf16_e256_k8_decode": W("bf16_e256_k8_decode", 37, 512, 256, 8, 384, None, "bf16"),
    "f32_e4_big_tiles": W("f32_e4_big_tiles", 600, 256, 4, 2, 384, 1.0, "f32"),
    "bf16_e3_k3": W("bf16_e3_k3", 333, 128, 3, 3, 256, None, "bf16"),
    # the ABI's maximum experts and slots per token, capacity-bound
    "bf16_e1024_k64_max": W("bf16_e1024_k64_max", 96, 128, 1024, 64, 128, 1.0, "bf16", 0.02),
    # one expert: every token takes it, the gate is exactly 1
    "f32_e1_k1": W("f32_e1_k1", 300, 128, 1, 1, 256, None, "f32"),
    # few, long down-GEMM tiles (32 stages): the down GEMM splits its reduction in two pieces
    "bf16_e8_split_down": W("bf16_e8_split_down", 700, 256, 8, 2, 2048, 1.25, "bf16", 1.1),
    "f32_e4_split_down": W("f32_e4_split_down", 600, 256, 4, 2, 1024, 1.0, "f32"),
    # a reduction of 64 stages over 8 m-tiles: the down GEMM splits it into four pieces
    "bf16_e8_split4_down": W("bf16_e8_split4_down", 700, 256, 8, 2, 4096, 1.25, "bf16", 1.1),
    # 320-row tiles where an expert's last tile (<= 128 rows) follows two or more full
    # tiles, so it runs double width over two n-tiles: kept rows [1085, 615] with an odd
    # n-tile count in the gate/up GEMM (F / 128 = 3) and a ragged one in the down GEMM
    # (d = 384); fp32 with [1004, 746]; and [997, 868, 737, 698] with the down GEMM split
    "bf16_e2_wide_tail": W("bf16_e2_wide_tail", 1700, 384, 2, 1, 384, None, "bf16", 0.6),
    "f32_e2_wide_tail": W("f32_e2_wide_tail", 1750, 256, 2, 1, 384, None, "f32", 0.4),
    "bf16_e4_wide_tail_split": W("bf16_e4_wide_tail_split", 1650, 256, 4, 2, 2048, None, "bf16",
                                 0.3),
    # 320-row tiles whose second 160-row band ends inside the expert's last rows with 1, 2,
    # 3, 4 and 5 live 32-row tiles (kept rows [568, 432, 313, 275, 205, 230, 187, 190]): the
    # band runs the k-loop copy that skips its empty tiles' MFMAs
    "bf16_e8_partial_bands": W("bf16_e8_partial_bands", 2400, 256, 8, 1, 384, None, "bf16",
                               0.4),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load_library()
    yield
    torch.cuda.synchronize()


def _i32(n, *shape):
    return torch.empty(shape if shape else (n,), dtype=torch.int32, device="cuda")


# ------------------------------------------------------------------------------- S2 routing
ROUTE_CASES = [(1000, 8, 2, "normal"), (37, 8, 1, "ties"), (513, 256, 8, "normal"),
               (300, 256, 8, "ties"), (64, 1000, 4, "normal"), (129, 3, 3, "ties"),
               (50, 1, 1, "normal"), (0, 8, 2, "normal"), (70, 64, 64, "ties"),
               (200, 1024, 64, "normal"),
               # the 16-lane row groups (E <= 256, k <= 16) at their edges: k = 16 slots,
               # E just past 16 and at 256, k past the lanes E alone would need, E = 2,
               # more tokens than the blocks' first pass; and the 64-lane groups just
               # outside them
               (333, 17, 16, "normal"), (100, 256, 16, "ties"), (77, 5, 5, "ties"),
               (90, 16, 9, "normal"), (91, 2, 2, "ties"), (2100, 256, 8, "normal"),
               (65, 257, 8, "normal")]


@pytest.mark.parametrize("T,E,k,kind", ROUTE_CASES)
def test_route_given_logits(T, E, k, kind):
    log(f"route T={T} E={E} k={k} {kind}")
    rng = np.random.default_rng(T * 7919 + E * 31 + k)
    if kind == "normal":
        L = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    else:
        L = rng.choice(np.array([-1.0, -0.0, 0.0, 0.5, 1.0], np.float32), size=(T, E))
    s = moe.shape(T, 128, E, k, 128, 0, moe.MOE_F32)
    logits = to_device(L, torch.float32)
    idx = _i32(0, T, k)
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    status = _i32(1)
    moe.route(s, None, None, None, logits, idx, w, status, logits_given=True)
    torch.cuda.synchronize()
    assert status.item() == 0
    if T == 0:
        return
    ref_idx = oracle.select_topk(L, k)
    ref_w = oracle.gate_weights(L, ref_idx)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    assert np.max(np.abs(w.cpu().numpy() - ref_w)) <= 1e-6


def test_route_nonfinite_logits_counted():
    T, E, k = 100, 16, 2
    rng = np.random.default_rng(5)
    L = rng.standard_normal((T, E)).astype(np.float32)
    bad_rows = [3, 17, 18, 99]
    L[3, 5] = np.nan
    L[17, 0] = np.inf
    L[18, 15] = -np.inf
    L[99, 7] = np.nan
    s = moe.shape(T, 128, E, k, 128, 0, moe.MOE_F32)
    idx, w, status = _i32(0, T, k), torch.empty((T, k), device="cuda"), _i32(1)
    moe.route(s, None, None, None, to_device(L, torch.float32), idx, w, status,
              logits_given=True)
    torch.cuda.synchronize()
    assert status.item() == len(bad_rows)
    good = np.setdiff1d(np.arange(T), bad_rows)
    ref_idx = oracle.select_topk(L[good], k)
    assert np.array_equal(idx.cpu().numpy()[good], ref_idx)


# ------------------------------------------------------------------------------- S1 logits
@pytest.mark.parametrize("name", ["tiny_f32", "bf16_e8_zipf_drops", "bf16_e256_k8_drops",
                                  "f32_e4_big_tiles"])
def test_router_logits(name):
    w = SMALL[name]
    log(f"logits {w}")
    h = host_inputs(w)
    dt = torch_dtype(w)
    s = shape_of(w)
    L = torch.empty((w.T, w.E), dtype=torch.float32, device="cuda")
    idx, gw = _i32(0, w.T, w.k), torch.empty((w.T, w.k), device="cuda")
    b = None if h["b_router"] is None else to_device(h["b_router"], torch.float32)
    moe.route(s, to_device(h["x"], dt), to_device(h["w_router"], dt), b, L, idx, gw)
    torch.cuda.synchronize()
    ref = oracle.router_logits(h["x"], h["w_router"], h["b_router"])
    err = float(np.max(np.abs(L.cpu().numpy() - ref)))
    log(f"  max|dL| = {err:.3e}, tol {logits_tol(ref):.3e}")
    assert err <= logits_tol(ref)


@pytest.mark.parametrize("T,d,E,dtype", [(2048, 256, 1024, "bf16"), (2047, 128, 1000, "f32"),
                                         (12300, 128, 100, "f32"), (6100, 256, 256, "bf16"),
                                         (600, 256, 1000, "bf16"), (1000, 128, 512, "bf16"),
                                         (300, 128, 40, "bf16"), (8200, 128, 40, "f32"),
                                         (12300, 128, 102, "bf16")])
def test_router_logits_tile_shapes(T, d, E, dtype):
    # sizes that select each router path: the expert-GEMM pipeline in dense mode (64 x 128
    # tiles, >= 192 of them; expert counts below one tile, at two tiles and ragged, ragged
    # token tails, and E = 102, whose rows do not start on 16-byte boundaries, so the
    # epilogue stores element by element), then the skinny kernel's 16 x 64 and 16 x 16
    # tiles
    log(f"router tiles T={T} d={d} E={E} {dtype}")
    rng = np.random.default_rng(T + E)
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    if dtype == "bf16":
        x, wr = (mi.bf16_bits_to_f32(mi.bf16_rne_np(a)) for a in (x, wr))
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    s = moe.shape(T, d, E, 1, 128, 0, moe.MOE_BF16 if dtype == "bf16" else moe.MOE_F32)
    L = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx, gw = _i32(0, T, 1), torch.empty((T, 1), device="cuda")
    moe.route(s, to_device(x, dt), to_device(wr, dt), to_device(b, torch.float32), L, idx, gw)
    torch.cuda.synchronize()
    ref = oracle.router_logits(x, wr, b)
    err = float(np.max(np.abs(L.cpu().numpy() - ref)))
    log(f"  max|dL| = {err:.3e}, tol {logits_tol(ref):.3e}")
    assert err <= logits_tol(ref)


# ------------------------------------------------------------------------------- S3-S5
DISPATCH_CASES = [
    # T, E, k, C, d, dtype, bias s
    (1000, 8, 2, 250, 256, "bf16", 0.8),
    (777, 8, 2, 0, 128, "f32", 0.0),
    (8192, 256, 8, 256, 128, "bf16", 0.05),
    (3, 3, 2, 1, 128, "f32", 0.0),
    (513, 5, 3, 100, 128, "bf16", 0.3),
    (2000, 1024, 64, 50, 128, "bf16", 0.01),
    (100, 1, 1, 40, 128, "f32", 0.0),
    (4096, 8, 2, 1280, 384, "bf16", 0.0),
    (1, 8, 8, 0, 128, "bf16", 0.0),
    # around the one-block dispatch's limits (2048 assignments, 256 experts): at the
    # assignments (one block), just past them (tiled), at both limits (one block), past
    # the experts (tiled); and tiled shapes whose scan also writes the tile table
    (1024, 8, 2, 280, 128, "bf16", 0.3),
    (1025, 8, 2, 280, 128, "bf16", 0.3),
    (256, 256, 8, 12, 128, "bf16", 0.05),
    (30, 257, 4, 0, 128, "f32", 0.0),
    (4097, 8, 2, 1100, 128, "bf16", 0.3),
    (1024, 256, 8, 40, 128, "bf16", 0.05),
]


def _run_dispatch(T, E, k, C, d, dtype, idx_np, x_np):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    s = moe.shape(T, d, E, k, 128, C, moe.MOE_BF16 if dtype == "bf16" else moe.MOE_F32)
    R = moe.max_rows(s)
    ws = torch.empty(moe.workspace_size(s), dtype=torch.uint8, device="cuda")
    out = dict(routed=_i32(E), kept=_i32(E), offsets=_i32(E + 1), src=_i32(R),
               dest=_i32(0, T, k), drops=_i32(k + 2),
               x_perm=torch.full((R, d), 7.0, dtype=dt, device="cuda"),
               slot=torch.full((R,), 7777, dtype=torch.int32, device="cuda"))
    moe.dispatch(s, to_device(idx_np, torch.int32), to_device(x_np, dt), ws, out["routed"],
                 out["kept"], out["offsets"], out["src"], out["dest"], out["drops"],
                 out["x_perm"], src_slot=out["slot"])
    torch.cuda.synchronize()
    return s, R, out


@pytest.mark.parametrize("T,E,k,C,d,dtype,bias", DISPATCH_CASES)
def test_dispatch_bit_exact(T, E, k, C, d, dtype, bias):
    log(f"dispatch T={T} E={E} k={k} C={C} d={d} {dtype}")
    rng = np.random.default_rng(T + 13 * E + 101 * k)
    L = rng.standard_normal((T, E)).astype(np.float32)
    L += (-bias * np.log(np.arange(1, E + 1))).astype(np.float32)[None, :]
    idx = oracle.select_topk(L, k)
    x = rng.standard_normal((T, d)).astype(np.float32)
    if dtype == "bf16":
        x = mi.bf16_bits_to_f32(mi.bf16_rne_np(x))
    s, R, g = _run_dispatch(T, E, k, C, d, dtype, idx, x)
    ref = oracle.dispatch(idx, E, C)
    N = ref["n_kept"]
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
    # the permutation is a pure copy: bit-exact
    xp = to_host(g["x_perm"][:N])
    assert np.array_equal(xp.view(np.uint32), oracle.permute(x, ref["src_token"], N).view(np.uint32))
    # conservation
    assert int(g["kept"].sum()) == T * k - int(drops[0])


def test_dispatch_zero_tokens():
    s, R, g = _run_dispatch(0, 8, 2, 10, 128, "bf16", np.zeros((0, 2), np.int32),
                            np.zeros((0, 128), np.float32))
    assert R == 0
    assert g["routed"].abs().sum().item() == 0 and g["kept"].abs().sum().item() == 0
    assert g["offsets"].abs().sum().item() == 0 and g["drops"].abs().sum().item() == 0


def test_dispatch_invalid_and_duplicate_ids():
    # Entries outside [0, E) are dropped; a token repeating an expert is still counted in
    # token-major order (the counting-sort definition).  Invalid ids are checked against the
    # oracle on a table where they are replaced by an extra expert E, whose rows are then
    # removed: the other experts' positions do not depend on it.
    T, E, k, C, d = 300, 6, 3, 40, 128
    rng = np.random.default_rng(77)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    inval = rng.random((T, k)) < 0.05
    idx_gpu = np.where(inval, np.where(rng.random((T, k)) < 0.5, -1, E), idx).astype(np.int32)
    idx_ref = np.where(inval, E, idx)
    x = rng.standard_normal((T, d)).astype(np.float32)
    s, R, g = _run_dispatch(T, E, k, C, d, "f32", idx_gpu, x)
    ref = oracle.dispatch(idx_ref, E + 1, C)
    assert np.array_equal(g["routed"].cpu().numpy(), ref["routed_counts"][:E])
    assert np.array_equal(g["kept"].cpu().numpy(), ref["tokens_per_expert"][:E])
    assert np.array_equal(g["offsets"].cpu().numpy(), ref["expert_offsets"][:E + 1])
    dest_ref = np.where(inval, -1, ref["dest_row"])
    assert np.array_equal(g["dest"].cpu().numpy(), dest_ref)
    drops = g["drops"].cpu().numpy()
    dropped = dest_ref < 0
    assert drops[0] == dropped.sum()
    assert np.array_equal(drops[1:k + 1], dropped.sum(0))
    assert drops[k + 1] == dropped.all(1).sum()


# ------------------------------------------------------------------------------- S6-S7
@pytest.mark.parametrize("name", ["tiny_f32", "bf16_e8_big_tiles", "bf16_e16_small_tiles",
                                  "bf16_e256_k8_decode", "f32_e4_big_tiles",
                                  "bf16_e8_zipf_drops", "bf16_e3_k3", "bf16_e2_wide_tail",
                                  "f32_e2_wide_tail", "bf16_e4_wide_tail_split",
                                  "bf16_e8_split4_down", "bf16_e8_partial_bands"])
def test_expert_ffn(name):
    w = SMALL[name]
    log(f"expert_ffn {w}")
    h = host_inputs(w)
    dt = torch_dtype(w)
    s = shape_of(w)
    C = s.capacity
    L = oracle.router_logits(h["x"], h["w_router"], h["b_router"])
    idx = oracle.select_topk(L, w.k)
    tab = oracle.dispatch(idx, w.E, C)
    N, R = tab["n_kept"], moe.max_rows(s)
    xp = np.zeros((R, w.d), np.float32)
    xp[:N] = oracle.permute(h["x"], tab["src_token"], N)
    ws = torch.empty(moe.workspace_size(s), dtype=torch.uint8, device="cuda")
    y = torch.zeros((R, w.d), dtype=dt, device="cuda")
    moe.expert_ffn(s, to_device(xp, dt), to_device(tab["expert_offsets"].astype(np.int32),
                                                   torch.int32),
                   to_device(h["w_gate"], dt), to_device(h["w_up"], dt),
                   to_device(h["w_down"], dt), ws, y)
    torch.cuda.synchronize()
    ref = oracle.expert_ffn(xp[:N], tab["expert_offsets"], h["w_gate"], h["w_up"], h["w_down"])
    err = rel_err(to_host(y[:N]), ref)
    log(f"  N={N} rel err {err:.3e}")
    assert err <= (1e-5 if w.dtype == "f32" else OUT_TOL)
    assert np.all(np.isfinite(to_host(y[:N])))


@pytest.mark.parametrize("name", ["bf16_e8_split_down", "f32_e4_split_down",
                                  "bf16_e8_split4_down", "bf16_e4_wide_tail_split"])
def test_split_down_deterministic(name):
    # A split down GEMM adds its pieces' fp32 partial-sum slots in slot order, so two runs
    # give the same bits; the second starts from a workspace of all-ones bytes (NaN floats
    # in every slot), which must not reach any kept row.
    w = SMALL[name]
    log(f"split down determinism {w}")
    h = host_inputs(w)
    dt = torch_dtype(w)
    s = shape_of(w)
    assert moe.workspace_size(s) > moe.workspace_layout(s)["down_acc"], "shape must split"
    L = oracle.router_logits(h["x"], h["w_router"], h["b_router"])
    tab = oracle.dispatch(oracle.select_topk(L, w.k), w.E, s.capacity)
    N, R = tab["n_kept"], moe.max_rows(s)
    xp = np.zeros((R, w.d), np.float32)
    xp[:N] = oracle.permute(h["x"], tab["src_token"], N)
    args = (to_device(xp, dt), to_device(tab["expert_offsets"].astype(np.int32), torch.int32),
            to_device(h["w_gate"], dt), to_device(h["w_up"], dt), to_device(h["w_down"], dt))
    ws = torch.zeros(moe.workspace_size(s), dtype=torch.uint8, device="cuda")
    ys = []
    for fill in (0, 255):
        ws.fill_(fill)
        y = torch.zeros((R, w.d), dtype=dt, device="cuda")
        moe.expert_ffn(s, *args, ws, y)
        torch.cuda.synchronize()
        ys.append(to_host(y[:N]))
    assert np.all(np.isfinite(ys[1]))
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32))


@pytest.mark.parametrize("name,pad", [("bf16_e8_big_tiles", False), ("bf16_e8_zipf_drops", False),
                                      ("bf16_e256_k8_decode", False), ("f32_e4_big_tiles", False),
                                      ("bf16_e8_zipf_drops", True), ("bf16_e3_k3", True)])
def test_gate_up_gathered_equals_packed(name, pad):
    # the GEMM that gathers x rows through src_token computes the same h, bit for bit, as
    # the GEMM over x_perm (same row values, same arithmetic), on the kept rows
    w = SMALL[name]
    log(f"gathered gate/up {w} pad={pad}")
    d_in = device_inputs(w)
    C = moe.capacity(w.T, w.k, w.E, w.capacity_factor)
    s = moe.shape(w.T, w.d, w.E, w.k, w.F, C, moe.MOE_BF16 if w.dtype == "bf16" else
                  moe.MOE_F32, flags=moe.MOE_FLAG_PAD_TO_CAPACITY if pad else 0)
    lay = moe.MoELayer(s)
    v = lay.view
    moe.route(s, d_in["x"], d_in["w_router"], d_in["b_router"], v("logits"), v("topk_idx"),
              v("topk_w"))
    moe.dispatch(s, v("topk_idx"), d_in["x"], lay.workspace, lay.routed_counts,
                 lay.tokens_per_expert, v("offsets"), v("src_token"), v("dest_row"), lay.drops,
                 v("x_perm"))
    moe.expert_gate_up(s, v("x_perm"), v("offsets"), d_in["w_gate"], d_in["w_up"],
                       lay.workspace, v("h"))
    h1 = v("h").clone()
    v("h").fill_(0)
    moe.expert_gate_up_gathered(s, d_in["x"], v("src_token"), v("offsets"), d_in["w_gate"],
                                d_in["w_up"], lay.workspace, v("h"))
    torch.cuda.synchronize()
    rows = torch.nonzero(v("src_token") >= 0).flatten()
    assert rows.numel() == int(lay.tokens_per_expert.sum())
    assert torch.equal(h1[rows], v("h")[rows])


@pytest.mark.parametrize("T,E,k,C", [(1000, 8, 2, 250), (1000, 8, 2, 0), (3001, 64, 6, 290)])
def test_dispatch_tables_only(T, E, k, C):
    # packed rows without a copy: every row slot past the kept rows must read -1 afterwards,
    # so the tables start out holding a sentinel
    d = 256
    rng = np.random.default_rng(21 + T + C)
    idx = oracle.select_topk(rng.standard_normal((T, E)).astype(np.float32), k)
    s = moe.shape(T, d, E, k, 128, C, moe.MOE_BF16)
    R = moe.max_rows(s)
    ws = torch.empty(moe.workspace_size(s), dtype=torch.uint8, device="cuda")
    g = dict(routed=_i32(E), kept=_i32(E), offsets=_i32(E + 1), src=_i32(R), dest=_i32(0, T, k),
             drops=_i32(k + 2))
    g["src"].fill_(0x5A5A5A5A)
    slot = torch.full((R,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    moe.dispatch(s, to_device(idx, torch.int32), None, ws, g["routed"], g["kept"], g["offsets"],
                 g["src"], g["dest"], g["drops"], None, src_slot=slot)
    torch.cuda.synchronize()
    ref = oracle.dispatch(idx, E, C)
    assert np.array_equal(g["dest"].cpu().numpy(), ref["dest_row"])
    assert np.array_equal(g["src"].cpu().numpy(), ref["src_token"][:R])
    assert np.array_equal(slot.cpu().numpy(), ref["src_slot"][:R])
    assert np.array_equal(g["offsets"].cpu().numpy(), ref["expert_offsets"])
    assert C == 0 or ref["expert_offsets"][-1] < R  # the capped cases leave a tail to mark


# ------------------------------------------------------------------------------- S8
@pytest.mark.parametrize("T,E,k,C,d,dtype", [(500, 8, 2, 110, 256, "bf16"),
                                             (300, 256, 8, 10, 128, "bf16"),
                                             (200, 4, 3, 0, 384, "f32")])
def test_combine(T, E, k, C, d, dtype):
    rng = np.random.default_rng(T + k)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    L = rng.standard_normal((T, E)).astype(np.float32)
    idx = oracle.select_topk(L, k)
    gates = oracle.gate_weights(L, idx).astype(np.float32)
    tab = oracle.dispatch(idx, E, C)
    s = moe.shape(T, d, E, k, 128, C, moe.MOE_BF16 if dtype == "bf16" else moe.MOE_F32)
    R = moe.max_rows(s)
    Y = rng.standard_normal((R, d)).astype(np.float32)
    if dtype == "bf16":
        Y = mi.bf16_bits_to_f32(mi.bf16_rne_np(Y))
    out = torch.empty((T, d), dtype=dt, device="cuda")
    moe.combine(s, to_device(Y, dt), to_device(tab["dest_row"].astype(np.int32), torch.int32),
                to_device(gates, torch.float32), out)
    torch.cuda.synchronize()
    ref = oracle.combine(Y, tab["dest_row"], gates)
    err = rel_err(to_host(out), ref)
    assert err <= (1e-6 if dtype == "f32" else 8e-3)  # one bf16 rounding of the sum
    full_drop = np.all(tab["dest_row"] < 0, axis=1)
    assert np.all(to_host(out)[full_drop] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dispatch_combine_identity_round_trip(dtype):
    # identity experts (y_perm = x_perm), k = 1, no capacity limit: out == x bit for bit
    T, E, k, d = 1000, 8, 1, 256
    rng = np.random.default_rng(11)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    L = rng.standard_normal((T, E)).astype(np.float32)
    idx = oracle.select_topk(L, k)
    x = rng.standard_normal((T, d)).astype(np.float32)
    if dtype == "bf16":
        x = mi.bf16_bits_to_f32(mi.bf16_rne_np(x))
    s, R, g = _run_dispatch(T, E, k, 0, d, dtype, idx, x)
    gates = torch.ones((T, k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, d), dtype=dt, device="cuda")
    moe.combine(s, g["x_perm"], g["dest"], gates, out)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out).view(np.uint32), x.view(np.uint32))


# ------------------------------------------------------------------------------- layer
def _layer_gpu(w, d_in, s):
    lay = moe.MoELayer(s)
    out = lay(d_in["x"], d_in["w_router"], d_in["b_router"], d_in["w_gate"], d_in["w_up"],
              d_in["w_down"])
    torch.cuda.synchronize()
    return lay, out


def check_layer_against_oracle(w, lay, h):
    """Compare one moe_layer result with the oracle run on the same seeded inputs: the
    logits against the oracle's float64 ones, the selection against the oracle's own
    routing up to near-ties, then, with the oracle routing from the GPU's fp32 logits, every
    routing table bit for bit and every output row (2e-2 * max|ref| in bf16, 1e-5 in fp32)."""
    s = lay.shape
    L_ref = oracle.router_logits(h["x"], h["w_router"], h["b_router"])
    L_gpu = lay.view("logits").cpu().numpy()
    tol = logits_tol(L_ref)
    assert float(np.max(np.abs(L_gpu - L_ref))) <= tol
    idx_gpu = lay.view("topk_idx").cpu().numpy()
    bad, unexplained = near_tie_ok(L_ref, idx_gpu, oracle.select_topk(L_ref, w.k), tol)
    assert not unexplained, f"selection differs beyond near-ties at tokens {unexplained[:10]}"
    res = oracle.moe_layer(h["x"], h["w_router"], h["b_router"], h["w_gate"], h["w_up"],
                           h["w_down"], w.k, s.capacity, logits=L_gpu)
    assert np.array_equal(idx_gpu, res["topk_idx"])
    assert np.max(np.abs(lay.view("topk_w").cpu().numpy() - res["topk_w"])) <= 1e-6
    assert np.array_equal(lay.routed_counts.cpu().numpy(), res["routed_counts"])
    assert np.array_equal(lay.tokens_per_expert.cpu().numpy(), res["tokens_per_expert"])
    assert np.array_equal(lay.view("dest_row").cpu().numpy(), res["dest_row"])
    assert np.array_equal(lay.view("src_token").cpu().numpy(),
                          res["src_token"][:moe.max_rows(s)])
    drops = lay.drops.cpu().numpy()
    assert drops[0] == res["drops_total"]
    assert np.array_equal(drops[1:w.k + 1], res["drops_per_slot"])
    assert drops[w.k + 1] == res["fully_dropped_tokens"]
    err = rel_err(to_host(lay.out), res["out"])
    tol_out = 1e-5 if w.dtype == "f32" else OUT_TOL
    log(f"  out rel err {err:.3e} over all {w.T} tokens (tol {tol_out:g}), "
        f"drops {int(drops[0])}, {len(bad)} near-tie tokens vs float64 logits")
    assert err <= tol_out
    return res


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_end_to_end(name):
    w = SMALL[name]
    log(f"layer {w}")
    h = host_inputs(w)
    s = shape_of(w)
    lay, _ = _layer_gpu(w, device_inputs(w), s)
    assert lay.status.item() == 0
    check_layer_against_oracle(w, lay, h)


def test_layer_deterministic():
    w = SMALL["bf16_e256_k8_drops"]
    s = shape_of(w)
    d_in = device_inputs(w)
    lay, out1 = _layer_gpu(w, d_in, s)
    N = int(lay.view("offsets")[-1])
    first = (out1.clone(), lay.view("dest_row").clone(), lay.view("h")[:N].clone(),
             lay.view("y_perm")[:N].clone())
    lay2, out2 = _layer_gpu(w, d_in, s)
    assert int(lay2.view("offsets")[-1]) == N
    assert torch.equal(first[0], out2)
    assert torch.equal(first[1], lay2.view("dest_row"))
    assert torch.equal(first[2], lay2.view("h")[:N])
    assert torch.equal(first[3], lay2.view("y_perm")[:N])


def test_layer_zero_tokens():
    w = W("zero", 0, 128, 8, 2, 128, 1.0, "bf16")
    s = shape_of(w, capacity=0)
    d_in = device_inputs(w)
    lay, _ = _layer_gpu(w, d_in, s)
    assert lay.routed_counts.abs().sum().item() == 0
    assert lay.drops.abs().sum().item() == 0 and lay.status.item() == 0


def test_device_generator_matches_host():
    w = SMALL["bf16_e8_zipf_drops"]
    for name in ("x", "w_gate", "w_down"):
        dev = to_host(mi.device_tensor(w, name))
        assert np.array_equal(dev, mi.host_tensor_f32(w, name))


# ------------------------------------------------------------------------------- graphs
@pytest.mark.parametrize("name,flags", [("bf16_e8_zipf_drops", 0), ("bf16_e256_k8_drops", 0),
                                        ("bf16_e8_zipf_drops", moe.MOE_FLAG_PAD_TO_CAPACITY)])
def test_layer_graph_replay_matches_eager(name, flags):
    # moe_layer only enqueues kernels (no allocation, memset or host synchronisation), so a
    # captured HIP graph replays it; every replay, with eager work of the program between
    # replays, must reproduce the eager result bit for bit
    w = SMALL[name]
    d_in = device_inputs(w)
    C = moe.capacity(w.T, w.k, w.E, w.capacity_factor)
    s = moe.shape(w.T, w.d, w.E, w.k, w.F, C, moe.MOE_BF16, flags=flags)
    args = (d_in["x"], d_in["w_router"], d_in["b_router"], d_in["w_gate"], d_in["w_up"],
            d_in["w_down"])
    eager = moe.MoELayer(s)
    eager(*args)
    torch.cuda.synchronize()
    lay = moe.MoELayer(s)
    lay(*args)  # warm-up outside the capture (kernel attributes are set on first use)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lay(*args)
    for rep in range(3):
        lay.out.fill_(0)
        lay.routed_counts.fill_(-1)
        eager(*args)  # eager work of the program between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lay.out, eager.out), f"replay {rep}"
        assert torch.equal(lay.routed_counts, eager.routed_counts)
        assert torch.equal(lay.drops, eager.drops)
        assert torch.equal(lay.view("dest_row"), eager.view("dest_row"))


# ------------------------------------------------------------------------------- streams
def test_layers_on_two_streams_match_one_stream():
    # Calls with distinct workspaces and outputs may run concurrently on different streams:
    # two layers of different shapes (one with decode-sized experts, one whose down GEMM
    # splits its reduction), enqueued alternately on two streams of default priority,
    # reproduce their one-stream results bit for bit.
    runs = []
    for name in ("bf16_e256_k8_drops", "bf16_e8_split_down"):
        w = SMALL[name]
        d_in = device_inputs(w)
        s = shape_of(w)
        args = (d_in["x"], d_in["w_router"], d_in["b_router"], d_in["w_gate"], d_in["w_up"],
                d_in["w_down"])
        ref = moe.MoELayer(s)
        ref(*args)
        runs.append((moe.MoELayer(s), ref, args))
    torch.cuda.synchronize()
    streams = (torch.cuda.Stream(), torch.cuda.Stream())
    for rep in range(3):
        for lay, _, _ in runs:
            lay.out.fill_(0)
            lay.routed_counts.fill_(-1)
        torch.cuda.synchronize()
        for _ in range(2):
            for (lay, _, args), st in zip(runs, streams):
                with torch.cuda.stream(st):
                    lay(*args)
        torch.cuda.synchronize()
        for lay, ref, _ in runs:
            assert torch.equal(lay.out, ref.out), f"rep {rep}"
            assert torch.equal(lay.routed_counts, ref.routed_counts)
            assert torch.equal(lay.drops, ref.drops)
            assert torch.equal(lay.view("dest_row"), ref.view("dest_row"))


def test_router_logits_past_grid_cap():
    # The router kernel's grid holds at most 2^16 token tiles of 16 tokens; the blocks
    # stride over the rest.  T = 2^20 + 77 tokens: blocks 0-5 also take tiles past 2^16.
    # The launch also clears the status word (pre-filled here), and one token with an
    # infinite input value is counted into it.
    T, d, E, k = (1 << 20) + 77, 128, 8, 2
    g = torch.Generator(device="cuda").manual_seed(12)
    x = torch.randn((T, d), generator=g, device="cuda").to(torch.bfloat16)
    x[T - 3, 5] = float("inf")
    wr = (torch.randn((E, d), generator=g, device="cuda") / d ** 0.5).to(torch.bfloat16)
    s = moe.shape(T, d, E, k, 128, 0, moe.MOE_BF16)
    L = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx, w = _i32(0, T, k), torch.empty((T, k), device="cuda")
    status = torch.full((1,), 77, dtype=torch.int32, device="cuda")
    moe.route(s, x, wr, None, L, idx, w, status)
    torch.cuda.synchronize()
    assert status.item() == 1
    wr_h = wr.float().cpu().numpy()
    for t0 in (0, (1 << 20) - 40, T - 90):
        rows = slice(t0, t0 + 80)
        xr = x[rows].float().cpu().numpy()
        ref = oracle.router_logits(xr, wr_h, None)
        got = L[rows].cpu().numpy()
        fin = np.all(np.isfinite(ref), axis=1)
        assert np.max(np.abs(got[fin] - ref[fin])) <= logits_tol(ref[fin])
        assert np.array_equal(idx[rows].cpu().numpy()[fin], oracle.select_topk(got[fin], k))
    assert not np.all(np.isfinite(L[T - 3].cpu().numpy()))


def test_route_given_logits_past_2_31_lanes():
    # The top-k kernel gives each token a group of G lanes (G = 64 for E >= 64): with
    # T = 2^25 + 1000 tokens, T * G passes 2^31, which 32-bit lane indices would wrap.
    # Tokens at both ends (and across the 2^31 boundary) must get the oracle's selection.
    T, E, k = (1 << 25) + 1000, 64, 1
    g = torch.Generator(device="cuda").manual_seed(11)
    logits = torch.randn((T, E), generator=g, device="cuda", dtype=torch.float32)
    s = moe.shape(T, 128, E, k, 128, 0, moe.MOE_F32)
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    status = _i32(1)
    moe.route(s, None, None, None, logits, idx, w, status, logits_given=True)
    torch.cuda.synchronize()
    assert status.item() == 0
    assert int((idx < 0).sum()) == 0  # every token written
    for t0 in (0, (1 << 25) - 500, T - 600):
        rows = slice(t0, t0 + 600)
        L = logits[rows].cpu().numpy()
        assert np.array_equal(idx[rows].cpu().numpy(), oracle.select_topk(L, k))
        assert np.all(w[rows].cpu().numpy() == 1.0)  # k = 1: the gate is exactly 1
    del logits
    torch.cuda.empty_cache()


def test_down_tail_split_whole_and_pieces():
    # A down GEMM with whole tiles and a split tail at a size the oracle runs in seconds:
    # T = 4096, k = 1, E = 8, no capacity limit plans 320-row tiles with at most 20 m-tiles
    # x 16 n-tiles (d = 4096) < two rounds, so the tail split is on (F = 2048: 32 stages,
    # two pieces).  The expert offsets are chosen so the table holds 20 m-tiles: 7 experts
    # of 330 rows (a full tile and a 10-row tail each) and one of 1786 (five full tiles and
    # a 186-row one): 320 tiles, 256 whole and 64 in two pieces each.  Outputs against the
    # oracle, and two runs bit for bit (the second from a NaN-filled workspace).
    T, d, E, k, F = 4096, 4096, 8, 1, 2048
    s = moe.shape(T, d, E, k, F, 0, moe.MOE_BF16)
    lay = moe.workspace_layout(s)
    assert moe.workspace_size(s) - lay["down_acc"] >= 128 * 320 * 256 * 4
    counts = np.array([330] * 7 + [T - 7 * 330])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    tiles = sum(-(-int(c) // 320) for c in counts)
    assert tiles == 20 and tiles * (d // 256) == 320
    rng = np.random.default_rng(77)
    bf = lambda a: mi.bf16_bits_to_f32(mi.bf16_rne_np(a.astype(np.float32)))  # noqa: E731
    xp = bf(rng.standard_normal((T, d)))
    wg = bf(rng.standard_normal((E, F, d)) / np.sqrt(d))
    wu = bf(rng.standard_normal((E, F, d)) / np.sqrt(d))
    wd = bf(rng.standard_normal((E, d, F)) / np.sqrt(d))
    args = (to_device(xp, torch.bfloat16), to_device(offsets, torch.int32),
            to_device(wg, torch.bfloat16), to_device(wu, torch.bfloat16),
            to_device(wd, torch.bfloat16))
    ws = torch.empty(moe.workspace_size(s), dtype=torch.uint8, device="cuda")
    ys = []
    for fill in (0, 255):
        ws.fill_(fill)
        y = torch.zeros((T, d), dtype=torch.bfloat16, device="cuda")
        moe.expert_ffn(s, *args, ws, y)
        torch.cuda.synchronize()
        ys.append(y)
    assert torch.equal(ys[0], ys[1])
    ref = oracle.expert_ffn(xp, offsets, wg, wu, wd)
    err = rel_err(to_host(ys[0]), ref)
    log(f"  down tail split (256 whole + 64 x 2 pieces): rel err {err:.3e}")
    assert err <= OUT_TOL


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_last_tile_heights_in_tall_plan(dtype):
    # Every kind of last row tile a 320-row plan runs, from explicit expert offsets: T = 3480,
    # k = 1, E = 12, no capacity limit gives a mean of 290 rows, which the plan covers with
    # one 320-row tile rather than two 256-row ones.  The counts put each boundary in a last
    # tile: 0, 1 and 128 rows (the 128-row tile), 129, 200 and 256 rows (the gate/up GEMM's
    # 256-row tile; the down GEMM keeps the 320-row one), 257 and 320 rows (a partly filled
    # and a full 320-row tile), 321 (a 1-row tail), 449 and 576 (129- and 256-row tails behind
    # one full tile), and 740 (a 100-row tail behind two full tiles: the double-width tile).
    # d = 384 leaves a half n-tile in the down GEMM.  Outputs against the oracle.
    T, d, E, k, F = 3480, 384, 12, 1, 512
    counts = np.array([128, 129, 256, 257, 320, 321, 449, 576, 0, 1, 200, 740])
    assert counts.sum() <= T * k
    mean = T * k // E
    r = mean + mean // 20
    assert -(-r // 320) < -(-r // 256)  # the plan takes the 320-row tile
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    s = moe.shape(T, d, E, k, F, 0, moe.MOE_BF16 if dtype == "bf16" else moe.MOE_F32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    rng = np.random.default_rng(91)
    if dtype == "bf16":
        cast = lambda a: mi.bf16_bits_to_f32(mi.bf16_rne_np(a.astype(np.float32)))  # noqa: E731
    else:
        cast = lambda a: a.astype(np.float32)  # noqa: E731
    xp = np.zeros((moe.max_rows(s), d), np.float32)
    xp[:N] = cast(rng.standard_normal((N, d)))
    wg = cast(rng.standard_normal((E, F, d)) / np.sqrt(d))
    wu = cast(rng.standard_normal((E, F, d)) / np.sqrt(d))
    wd = cast(rng.standard_normal((E, d, F)) / np.sqrt(F))
    ws = torch.empty(moe.workspace_size(s), dtype=torch.uint8, device="cuda")
    y = torch.zeros((xp.shape[0], d), dtype=tdt, device="cuda")
    log(f"last tile heights {dtype}: counts {counts.tolist()}")
    moe.expert_ffn(s, to_device(xp, tdt), to_device(offsets, torch.int32), to_device(wg, tdt),
                   to_device(wu, tdt), to_device(wd, tdt), ws, y)
    torch.cuda.synchronize()
    ref = oracle.expert_ffn(xp[:N], offsets, wg, wu, wd)
    out = to_host(y[:N])
    assert np.all(np.isfinite(out))
    tol = 1e-5 if dtype == "f32" else OUT_TOL
    for e in range(E):  # per expert, so a wrong tile path names its expert
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            err = rel_err(out[lo:hi], ref[lo:hi])
            assert err <= tol, (e, int(counts[e]), err)
    log(f"  rel err {rel_err(out, ref):.3e}")
