"""The C-ABI library on the host: it loads, exports every declared entry point, and its host
logic (capacity, row bound, workspace layout, argument validation) behaves as documented.
Nothing here launches a kernel: every call below is rejected before the first HIP call."""
import ctypes

import numpy as np
import pytest

import oracle
import routing_expert_ffn_router_amd as moe

lib = moe.load_library()


def test_exports_every_declared_function():
    names = moe.header_functions()
    assert {"moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_layer"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_calib_library_exports_its_header():
    # the MFMA-rate calibration of the measurement harness lives in libmoe_calib.so
    import os

    calib = moe.load_calib()
    names = moe.header_functions(os.path.join(os.path.dirname(moe.HEADER_PATH),
                                              "moe_calib.h"))
    assert names == ["moe_calib_mfma", "moe_calib_wall_clock_khz"]
    for n in names:
        assert hasattr(calib, n), n
    # invalid arguments are refused before any HIP call
    sink = ctypes.c_void_p(16)
    for blocks, iters, operands, shape in [(0, 1, 1, 0), (1, 0, 1, 0), (1, 1, 2, 0),
                                           (-1, 5, 0, 1), (1, 1, 1, 2), (1, 1, 0, -1)]:
        assert calib.moe_calib_mfma(blocks, iters, 0, operands, shape, sink, sink, None) == -1
    assert calib.moe_calib_mfma(1, 1, 0, 1, 0, None, sink, None) == -1
    assert calib.moe_calib_mfma(1, 1, 0, 1, 1, sink, None, None) == -1
    assert calib.moe_calib_wall_clock_khz(None) == -1


def test_header_cites_the_pages():
    text = " ".join(open(moe.HEADER_PATH).read().replace("*", " ").split())
    for section in ("Deep dive", "Technical details", "Capacity factor changes quality",
                    "All-to-all must be profiled separately from compute"):
        assert section in text


@pytest.mark.parametrize("T", [0, 1, 7, 64, 100, 2048, 4096, 8192, 25, 80, 333])
@pytest.mark.parametrize("k,E", [(1, 4), (2, 8), (8, 256), (3, 5), (8, 4)])
@pytest.mark.parametrize("cf", [0.5, 1.0, 1.1, 1.25, 2.0, 3.3, None])
def test_capacity_matches_oracle(T, k, E, cf):
    if k > E:
        return
    assert moe.capacity(T, k, E, cf) == oracle.capacity(T, k, E, cf)


def test_capacity_invalid():
    assert lib.moe_capacity(-1, 2, 8, 1.0) == -1
    assert lib.moe_capacity(10, 0, 8, 1.0) == -1
    assert lib.moe_capacity(10, 2, 8, float("nan")) == -1
    assert lib.moe_capacity(10, 2, 8, -1.0) == 0


def test_max_rows_and_workspace():
    s = moe.shape(4096, 4096, 8, 2, 14336, 1280)
    assert moe.max_rows(s) == 8192
    s2 = moe.shape(2048, 6144, 8, 2, 16384, 640)
    assert moe.max_rows(s2) == 4096
    s3 = moe.shape(256, 7168, 256, 8, 2048, 0)
    assert moe.max_rows(s3) == 2048
    s4 = moe.shape(100, 128, 8, 2, 128, 5)
    assert moe.max_rows(s4) == 40  # E * C < T * k
    lay = moe.workspace_layout(s)
    offs = [lay[n] for n in moe.WS_REGIONS]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    total = moe.workspace_size(s)
    R, d, F = 8192, 4096, 14336
    assert total >= lay["y_perm"] + R * d * 2
    assert lay["h"] - lay["x_perm"] >= R * d * 2
    assert lay["y_perm"] - lay["h"] >= R * F * 2


def _down_acc_bytes(s):
    return moe.workspace_size(s) - moe.workspace_layout(s)["down_acc"]


def test_down_split_region():
    # Tail split of the down GEMM: when t = m-tiles (upper bound) x ceil(d / 256) is below
    # two rounds of 256 CUs, the tiles of the last partial round (counted on the device)
    # split their reduction into up to S = min(8, stages / 16) pieces, stages = F * elt /
    # 128, S >= 2.  The workspace then ends with min(256, t * S) slots of BM x 256 fp32
    # partial sums (BM = 320 or 256, the plan's row tile).
    # Mixtral-8x22B-shaped, C = 640, 320-row tiles: t <= 16 x 24 = 384, 256 stages -> S = 8,
    # 256 slots
    s = moe.shape(2048, 6144, 8, 2, 16384, 640)
    assert _down_acc_bytes(s) == 256 * 320 * 256 * 4
    # Mixtral-8x7B-shaped: t <= 32 x 16 = 512 = 2 rounds -> no split
    assert _down_acc_bytes(moe.shape(4096, 4096, 8, 2, 14336, 1280)) == 0
    # decode-sized experts stream weights: never split
    assert _down_acc_bytes(moe.shape(256, 7168, 256, 8, 2048, 0)) == 0
    # DeepSeek-V3 mixed batch: t = 256 x 28 = 28 rounds -> no split
    assert _down_acc_bytes(moe.shape(8192, 7168, 256, 8, 2048, 256)) == 0
    # a short reduction (F * 2 / 128 = 6 stages) does not split; 32 stages allow two
    # pieces, 64 stages four (t <= 8 m-tiles of 256 rows x 1)
    assert _down_acc_bytes(moe.shape(700, 256, 8, 2, 384, 219)) == 0
    assert _down_acc_bytes(moe.shape(700, 256, 8, 2, 2048, 219)) == 8 * 2 * 256 * 256 * 4
    assert _down_acc_bytes(moe.shape(700, 256, 8, 2, 4096, 219)) == 8 * 4 * 256 * 256 * 4
    # fp32: 4-byte elements, F = 1024 is 32 stages (two pieces of t <= 4 tiles of 320 rows);
    # F = 896 is 28 -> none
    assert _down_acc_bytes(moe.shape(600, 256, 4, 2, 1024, 300, moe.MOE_F32)) == \
        4 * 2 * 320 * 256 * 4
    assert _down_acc_bytes(moe.shape(600, 256, 4, 2, 896, 300, moe.MOE_F32)) == 0


BAD_SHAPES = [
    (dict(T=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(k=9), moe.MOE_ERR_INVALID_ARG),
    (dict(k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(E=0), moe.MOE_ERR_INVALID_ARG),
    (dict(d=100), moe.MOE_ERR_UNSUPPORTED),
    (dict(F=200), moe.MOE_ERR_UNSUPPORTED),
    (dict(dtype=7), moe.MOE_ERR_UNSUPPORTED),
    (dict(E=2048, k=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(E=128, k=65), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=1 << 30, k=2), moe.MOE_ERR_UNSUPPORTED),
    # variant fields
    (dict(flags=8), moe.MOE_ERR_INVALID_ARG),
    (dict(flags=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(n_groups=0, topk_groups=1), moe.MOE_ERR_INVALID_ARG),
    (dict(n_groups=-2, topk_groups=1), moe.MOE_ERR_INVALID_ARG),
    (dict(n_groups=3, topk_groups=1), moe.MOE_ERR_INVALID_ARG),       # 3 does not divide 8
    (dict(n_groups=4, topk_groups=0), moe.MOE_ERR_INVALID_ARG),
    (dict(n_groups=4, topk_groups=5), moe.MOE_ERR_INVALID_ARG),
    (dict(n_groups=8, topk_groups=1, k=2), moe.MOE_ERR_INVALID_ARG),  # k > 1 group of 1
    (dict(E=256, k=2, n_groups=128, topk_groups=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=1 << 22, E=1024, k=1, capacity=0, flags=1), moe.MOE_ERR_UNSUPPORTED),  # E*C
    # a grouped-GEMM grid past 2^32 threads: 2^25 rows of one expert x 2^20 columns
    (dict(T=1 << 25, E=1, k=1, F=1 << 20, capacity=0), moe.MOE_ERR_UNSUPPORTED),
]


def _shape(**kw):
    base = dict(T=64, d=128, E=8, k=2, F=256, capacity=32, dtype=moe.MOE_F32, flags=0,
                n_groups=0, topk_groups=0)
    base.update(kw)
    return moe.shape(base["T"], base["d"], base["E"], base["k"], base["F"], base["capacity"],
                     base["dtype"], base["flags"], base["n_groups"], base["topk_groups"])


FAKE = 1 << 40  # an aligned address that is never dereferenced: calls fail validation first


@pytest.mark.parametrize("kw,err", BAD_SHAPES)
def test_bad_shapes_rejected_everywhere(kw, err):
    s = ctypes.byref(_shape(**kw))
    p = FAKE
    assert lib.moe_workspace_size(s) == 0
    assert lib.moe_max_rows(s) == -1
    assert lib.moe_route(s, p, p, None, p, 0, p, p, None, None) == err
    assert lib.moe_dispatch(s, p, p, p, 1 << 40, p, p, p, p, None, p, p, p, None) == err
    assert lib.moe_expert_ffn(s, p, p, p, p, p, p, 1 << 40, p, None) == err
    assert lib.moe_combine(s, p, p, p, p, None) == err
    assert lib.moe_slot_counts(s, p, p, p, p, None) == err
    assert lib.moe_expert_gate_up_gathered(s, p, p, p, p, p, p, 1 << 40, p, None) == err
    assert lib.moe_layer(s, p, p, None, p, p, p, p, 1 << 40, p, None, None, None, None,
                         None) == err


GOOD_VARIANTS = [dict(flags=moe.MOE_FLAG_PAD_TO_CAPACITY), dict(flags=moe.MOE_FLAG_SLOT_MAJOR),
                 dict(flags=moe.MOE_FLAG_BIAS_SELECTION_ONLY), dict(flags=7),
                 dict(n_groups=4, topk_groups=1), dict(n_groups=4, topk_groups=4),
                 dict(n_groups=1, topk_groups=0), dict(n_groups=8, topk_groups=2),
                 dict(E=256, k=8, n_groups=64, topk_groups=4)]


@pytest.mark.parametrize("kw", GOOD_VARIANTS)
def test_variant_shapes_accepted(kw):
    sh = _shape(**kw)
    assert moe.workspace_size(sh) > 0 and moe.max_rows(sh) > 0


def test_pad_to_capacity_rows_and_workspace():
    for C, want in ((32, 8 * 32), (0, 8 * 64), (100, 8 * 64)):  # C > T means C = T
        packed = _shape(capacity=C)
        padded = _shape(capacity=C, flags=moe.MOE_FLAG_PAD_TO_CAPACITY)
        assert moe.max_rows(padded) == want
        assert moe.max_rows(packed) == min(64 * 2, want)
        lay = moe.workspace_layout(padded)
        assert lay["h"] - lay["x_perm"] >= want * 128 * 4
    # C = 8: padded rows E*C = 64 are fewer than T*k = 128 packed row slots
    assert moe.max_rows(_shape(capacity=8, flags=1)) == 64 == moe.max_rows(_shape(capacity=8))


def test_gathered_gate_up_checks():
    s = ctypes.byref(_shape())
    p = FAKE
    f = lib.moe_expert_gate_up_gathered
    assert f(s, p, None, p, p, p, p, 1 << 40, p, None) == moe.MOE_ERR_INVALID_ARG  # src_token
    assert f(s, None, p, p, p, p, p, 1 << 40, p, None) == moe.MOE_ERR_INVALID_ARG  # x
    assert f(s, p + 8, p, p, p, p, p, 1 << 40, p, None) == moe.MOE_ERR_ALIGNMENT
    assert f(s, p, p, p, p, p, None, 1 << 40, p, None) == moe.MOE_ERR_WORKSPACE
    big = _shape(T=1 << 20, d=1 << 11, k=1, dtype=moe.MOE_BF16)  # x is 4 GiB: no 32-bit rows
    assert f(ctypes.byref(big), p, p, p, p, p, p, 1 << 40, p, None) == moe.MOE_ERR_UNSUPPORTED
    assert not moe.gathered_layer(big) and moe.gathered_layer(_shape())
    assert not moe.gathered_layer(_shape(flags=moe.MOE_FLAG_PAD_TO_CAPACITY))


def test_dispatch_tables_only_accepts_null_x_perm():
    s = ctypes.byref(_shape())
    p = FAKE
    # x_perm NULL: x is not needed either; the call fails only at the workspace check
    assert lib.moe_dispatch(s, p, None, p, 16, p, p, p, p, None, p, p, None, None) == \
        moe.MOE_ERR_WORKSPACE
    # x_perm given without x
    assert lib.moe_dispatch(s, p, None, p, 1 << 40, p, p, p, p, None, p, p, p, None) == \
        moe.MOE_ERR_INVALID_ARG


def test_slot_counts_null_outputs_rejected():
    s = ctypes.byref(_shape())
    p = FAKE
    assert lib.moe_slot_counts(s, p, p, None, p, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_slot_counts(s, None, p, p, p, None) == moe.MOE_ERR_INVALID_ARG


def test_routing_record_from_counts_matches_oracle():
    # host summary of per-slot counts against the oracle's record built from the routing
    import oracle

    rng = np.random.default_rng(7)
    T, E, k, C = 300, 16, 4, 70
    L = (rng.standard_normal((T, E)) - 0.5 * np.log(np.arange(1, E + 1))).astype(np.float32)
    idx = oracle.select_topk(L, k)
    tab = oracle.dispatch(idx, E, C)
    rbs = np.zeros((k, E), np.int64)
    kbs = np.zeros((k, E), np.int64)
    for j in range(k):
        np.add.at(rbs[j], idx[:, j], 1)
        np.add.at(kbs[j], idx[:, j][tab["dest_row"][:, j] >= 0], 1)
    pl = np.arange(E) % 4
    got = moe.routing_record(T, rbs, kbs, pl, ranks_per_node=2)
    want = oracle.routing_record(idx, tab["dest_row"], E, pl, ranks_per_node=2)
    for key, v in want.items():
        if isinstance(v, list) and v and isinstance(v[0], list):
            assert got[key] == v, key
        else:
            assert got[key] == pytest.approx(v), key


def test_null_shape():
    assert lib.moe_route(None, FAKE, FAKE, None, FAKE, 0, FAKE, FAKE, None, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert lib.moe_workspace_size(None) == 0


def test_null_pointers_rejected():
    s = ctypes.byref(_shape())
    p = FAKE
    E = moe.MOE_ERR_INVALID_ARG
    assert lib.moe_route(s, None, p, None, p, 0, p, p, None, None) == E  # x
    assert lib.moe_route(s, p, p, None, None, 0, p, p, None, None) == E  # logits
    assert lib.moe_dispatch(s, None, p, p, 1 << 40, p, p, p, p, None, p, p, p, None) == E
    assert lib.moe_dispatch(s, p, p, p, 1 << 40, None, p, p, p, None, p, p, p, None) == E
    assert lib.moe_expert_ffn(s, p, p, None, p, p, p, 1 << 40, p, None) == E
    assert lib.moe_combine(s, p, None, p, p, None) == E
    assert lib.moe_layer(s, p, None, None, p, p, p, p, 1 << 40, p, None, None, None, None,
                         None) == E


def test_misaligned_pointers_rejected():
    s = ctypes.byref(_shape())
    p, q = FAKE, FAKE + 8
    A = moe.MOE_ERR_ALIGNMENT
    assert lib.moe_route(s, q, p, None, p, 0, p, p, None, None) == A
    assert lib.moe_dispatch(s, p, p, p, 1 << 40, p, p, p, p, None, p, p, q, None) == A
    assert lib.moe_expert_ffn(s, p, p, p, q, p, p, 1 << 40, p, None) == A
    assert lib.moe_combine(s, q, p, p, p, None) == A
    assert lib.moe_layer(s, p, p, None, p, p, p, p, 1 << 40, q, None, None, None, None,
                         None) == A
    # the workspace must be 256-byte aligned
    assert lib.moe_dispatch(s, p, p, p + 16, 1 << 40, p, p, p, p, None, p, p, p, None) == A


def test_workspace_checked():
    sh = _shape()
    s = ctypes.byref(sh)
    p = FAKE
    need = moe.workspace_size(sh)
    W = moe.MOE_ERR_WORKSPACE
    assert lib.moe_dispatch(s, p, p, None, need, p, p, p, p, None, p, p, p, None) == W
    assert lib.moe_dispatch(s, p, p, p, need - 1, p, p, p, p, None, p, p, p, None) == W
    assert lib.moe_expert_ffn(s, p, p, p, p, p, p, need - 256, p, None) == W
    assert lib.moe_layer(s, p, p, None, p, p, p, p, 16, p, None, None, None, None, None) == W


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5, 42):
        assert isinstance(moe.status_string(st), str)
    assert moe.status_string(-4).startswith("workspace")


def test_library_has_no_oracle_or_torch_dependency():
    # the product library is self-contained HIP code: no Python, no torch symbols
    import subprocess

    out = subprocess.run(["ldd", moe.LIB_PATH], capture_output=True, text=True).stdout
    assert "torch" not in out and "python" not in out.lower()
    assert "amdhip64" in out


# ---------------------------------------------------------------- S9 record (host C code)
def _stats_cases():
    rng = np.random.default_rng(11)
    cases = []
    for E in (1, 2, 4, 8, 20, 40, 100, 256, 1000, 1024):
        for k in (1, 2, 8):
            if k > E:
                continue
            T = int(rng.integers(1, 3000))
            idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if E <= 40 else \
                rng.integers(0, E, (T, k))
            n = np.bincount(idx.ravel(), minlength=E)
            cases.append((T, k, n))
    return cases


@pytest.mark.parametrize("T,k,n", _stats_cases())
def test_expert_stats_matches_oracle(T, k, n):
    C = max(1, int(np.median(n)))
    c = np.minimum(n, C)
    got = moe.expert_stats(T, k, n, c)
    want = oracle.expert_stats(n, T, k, tokens_per_expert=c, dropped=int((n - c).sum()))
    for key in ("active_tokens", "top_k", "expert_p50", "expert_p95", "expert_max",
                "dropped_tokens"):
        assert got[key] == want[key], key
    assert got["expert_mean"] == pytest.approx(want["expert_mean"], rel=1e-15)
    assert got["expert_max_to_mean"] == pytest.approx(want["expert_max_to_mean"], rel=1e-15)
    assert got["routed"] == n.sum() and got["experts"] == n.size
    # conservation: kept rows plus dropped assignments are the routed ones
    assert got["kept_rows"] + got["dropped_tokens"] == got["routed"]
    assert got["active_experts"] == int((c > 0).sum())
    # the top-5 % share agrees with the oracle's routing record of the same counts
    top = int(np.ceil(0.05 * n.size))
    assert got["top_5_percent_experts"] == top
    assert got["top_5_percent_expert_share"] == pytest.approx(
        np.sort(n)[::-1][:top].sum() / n.sum(), rel=1e-15)


def test_expert_stats_page_example():
    # [EP-checks] "Mean expert load proves almost nothing": its printed record fixes max
    # and max/mean of the four counts (1003 / 882.25 -> 1.14); its p50 / p95 fit no standard
    # percentile rule and are not pins
    import json
    import os

    rec = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                      "expert_stats_record.json")))
    n = np.array(rec["tokens_per_expert"])
    st = moe.expert_stats(int(n.sum()) // 2, rec["top_k"], n)
    assert st["expert_max"] == rec["expert_max"]
    assert round(st["expert_max_to_mean"], 2) == rec["expert_max_to_mean"]
    assert st["dropped_tokens"] == rec["dropped_tokens"] == 0
    # nearest rank on 1..100: the median is 50 and the 95th percentile 95
    st = moe.expert_stats(5050, 1, np.arange(1, 101))
    assert (st["expert_p50"], st["expert_p95"], st["expert_max"]) == (50, 95, 100)


def test_expert_stats_degenerate_and_invalid():
    st = moe.expert_stats(0, 2, np.zeros(8, np.int32))
    assert st["routed"] == 0 and st["top_5_percent_expert_share"] == 0.0
    assert np.isnan(st["expert_max_to_mean"])
    with pytest.raises(moe.MoeError):
        moe.expert_stats(10, 2, np.array([3, -1]))
    with pytest.raises(moe.MoeError):
        moe.expert_stats(10, 2, np.array([3, 1]), np.array([4, 1]))  # kept > routed
    with pytest.raises(moe.MoeError):
        moe.placement_load(np.array([3, 1]), np.array([0, 2]), n_ranks=2)  # rank 2 of 2


# ---------------------------------------------------------------- memory by phase
PHASE_SHAPES = [
    _shape(),                                                  # packed: the GEMM gathers
    _shape(flags=moe.MOE_FLAG_PAD_TO_CAPACITY),                # padded: x_perm is copied
    moe.shape(2048, 6144, 8, 2, 16384, 640),                   # down GEMM split in three
    moe.shape(256, 7168, 256, 8, 2048, 0),                     # decode-sized
    moe.shape(1 << 20, 2048, 8, 1, 128, 0, moe.MOE_BF16),      # x past 2^31 bytes: copied
    _shape(T=0),
]


@pytest.mark.parametrize("sh", PHASE_SHAPES)
def test_workspace_phases_follow_the_layout(sh):
    # [EP-checks] "Memory must be counted by phase": the bytes each phase has written are
    # the sizes of the regions its stages write, read off moe_workspace_layout
    ph = moe.workspace_phases(sh)
    lay = moe.workspace_layout(sh)
    total = moe.workspace_size(sh)
    names = moe.WS_REGIONS
    ends = [lay[names[i + 1]] if i + 1 < len(names) else total for i in range(len(names))]
    R = moe.max_rows(sh)
    b = 2 if sh.dtype == moe.MOE_BF16 else 4
    size = {
        "logits": sh.T * sh.E * 4, "topk_idx": sh.T * sh.k * 4, "topk_w": sh.T * sh.k * 4,
        "routed": sh.E * 4, "kept": sh.E * 4, "offsets": (sh.E + 1) * 4, "src_token": R * 4,
        "dest_row": sh.T * sh.k * 4, "drops": (sh.k + 2) * 4, "status": 4,
        "x_perm": R * sh.d * b, "h": R * sh.F * b, "y_perm": R * sh.d * b,
    }
    # region sizes bounded by the layout: each region ends before the next one starts
    for i, n in enumerate(names):
        room = ends[i] - lay[n]
        if n in size:
            assert size[n] <= room < size[n] + 256, n
    internal = {n: ends[i] - lay[n] for i, n in enumerate(names)
                if n in ("tile_hist", "tile_base", "sched", "down_acc")}
    pack = sum(size[n] for n in ("logits", "topk_idx", "topk_w", "status", "routed", "kept",
                                 "offsets", "src_token", "dest_row", "drops"))
    # the dispatch writes the GEMMs' tile table, and its per-tile tables when it runs tiled
    pack_internal = internal["sched"] + internal["tile_hist"] + internal["tile_base"]
    if not moe.gathered_layer(sh):
        pack += size["x_perm"]
    assert ph["before_layer"] == 0
    assert pack <= ph["after_pack"] <= pack + pack_internal
    assert ph["after_dispatch"] == ph["after_pack"]
    if sh.T == 0:
        assert ph["after_experts"] == ph["after_pack"]
        return
    exp = size["h"] + size["y_perm"]
    grown = ph["after_experts"] - ph["after_pack"]
    assert exp <= grown <= exp + internal["down_acc"]
    assert ph["after_experts"] <= total
    if sh.E == 8 and sh.T == 2048:  # the split down GEMM's fp32 slots are counted
        assert grown >= exp + 256 * 320 * 256 * 4


def test_no_workspace_dispatch_checks_before_any_launch():
    # argument checks as moe_dispatch; a shape whose two scratch tables exceed the static
    # array is refused with MOE_ERR_SCRATCH before the first HIP call
    p = FAKE
    f = lib.moe_dispatch_no_workspace
    big = _shape(T=1 << 21, E=1024, k=1, capacity=0)  # 2 x 4096 x 1024 x 4 B = 32 MiB
    assert f(ctypes.byref(big), p, None, p, p, p, p, None, p, p, None, None) == \
        moe.MOE_ERR_SCRATCH
    s = ctypes.byref(_shape())
    assert f(s, None, p, p, p, p, p, None, p, p, None, None) == moe.MOE_ERR_INVALID_ARG
    assert f(s, p, p, p, p, p, p, None, p, p, p + 8, None) == moe.MOE_ERR_ALIGNMENT
    assert f(ctypes.byref(_shape(k=9)), p, p, p, p, p, p, None, p, p, None, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert moe.status_string(moe.MOE_ERR_SCRATCH).startswith("shape needs more")
