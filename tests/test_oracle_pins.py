"""Pins of the CPU oracle to facts outside itself.

Each test checks the oracle against one of: brute force over tiny inputs, a closed form,
an invariant of the method, a special case that reduces to a library routine, or a value
printed on the pages (tests/golden/, each with its source).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


# ---------------------------------------------------------------- S1 router logits
def test_logits_unit_rows_pick_weight_columns():
    E, d = 5, 7
    W = rng.standard_normal((E, d))
    b = rng.standard_normal(E).astype(np.float32)
    X = np.eye(d)  # token t is the unit vector e_t
    L = oracle.router_logits(X, W, b)
    assert L.dtype == np.float32
    want = (W.T + b.astype(np.float64)[None, :]).astype(np.float32)  # L[t, e] = W[e, t] + b[e]
    assert np.array_equal(L, want)


def test_logits_integer_inputs_exact():
    # small integers: every product and sum is exact in float64 and in float32
    x = rng.integers(-8, 9, size=(6, 10)).astype(np.float64)
    W = rng.integers(-8, 9, size=(4, 10)).astype(np.float64)
    L = oracle.router_logits(x, W)
    brute = np.array([[sum(x[t, i] * W[e, i] for i in range(10)) for e in range(4)]
                      for t in range(6)], dtype=np.float32)
    assert np.array_equal(L, brute)


# ---------------------------------------------------------------- S2 selection
def _brute_topk(row, k):
    """The k-subset that beats every outside expert under (value desc, index asc)."""
    E = len(row)

    def better(a, b):  # a strictly before b
        return row[a] > row[b] or (row[a] == row[b] and a < b)

    winners = [S for S in itertools.combinations(range(E), k)
               if all(better(s, o) for s in S for o in range(E) if o not in S)]
    assert len(winners) == 1
    S = list(winners[0])
    # order inside the subset: repeatedly take the element that beats all the others
    out = []
    while S:
        top = [s for s in S if all(better(s, o) for o in S if o != s)]
        assert len(top) == 1
        out.append(top[0])
        S.remove(top[0])
    return out


@pytest.mark.parametrize("E", [3, 4])
def test_topk_brute_force_on_tie_grid(E):
    vals = np.array([-1.0, -0.0, 0.0, 1.0], dtype=np.float32)
    rows = np.array(list(itertools.product(vals, repeat=E)), dtype=np.float32)
    for k in range(1, E + 1):
        got = oracle.select_topk(rows, k)
        for t in range(rows.shape[0]):
            assert list(got[t]) == _brute_topk(rows[t], k), (rows[t], k)


def test_topk_random_brute_force():
    L = rng.integers(-3, 4, size=(300, 6)).astype(np.float32) * np.float32(0.5)
    for k in (1, 2, 3, 6):
        got = oracle.select_topk(L, k)
        for t in range(L.shape[0]):
            assert list(got[t]) == _brute_topk(L[t], k)


def test_gates_k1_is_one_and_sum_is_one():
    L = rng.standard_normal((200, 16)).astype(np.float32) * 3
    idx = oracle.select_topk(L, 1)
    w1 = oracle.gate_weights(L, idx)
    assert np.all(w1 == 1.0)
    for k in (2, 5, 16):
        w = oracle.gate_weights(L, oracle.select_topk(L, k))
        assert np.all(np.abs(w.sum(axis=1) - 1.0) < 1e-12)
        assert np.all(np.diff(w, axis=1) <= 0)  # slot order is best first


def test_gates_k_equals_E_is_softmax():
    L = rng.standard_normal((64, 8)).astype(np.float32) * 4
    idx = oracle.select_topk(L, 8)
    w = oracle.gate_weights(L, idx)
    sm = torch.softmax(torch.from_numpy(L.astype(np.float64)), dim=1).numpy()
    want = np.take_along_axis(sm, idx.astype(np.int64), axis=1)
    assert np.max(np.abs(w - want)) < 1e-14


def test_gates_are_softmax_ratio():
    # renormalised gate = p_e / sum_sel p with p the full softmax (denominator cancels)
    L = rng.standard_normal((50, 12)).astype(np.float32)
    idx = oracle.select_topk(L, 3)
    p = torch.softmax(torch.from_numpy(L.astype(np.float64)), dim=1).numpy()
    ps = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    assert np.max(np.abs(oracle.gate_weights(L, idx) - ps / ps.sum(1, keepdims=True))) < 1e-14


# ---------------------------------------------------------------- S4 capacity
def test_capacity_worked_values():
    # C = mean tokens per expert (T*k/E) times the capacity factor, worked by hand
    assert oracle.capacity(64, 2, 8, 2.0) == 32  # 64*2/8 = 16, x2
    assert oracle.capacity(4096, 2, 8, 1.25) == 1280  # 1024 x 1.25
    assert oracle.capacity(2048, 2, 8, 1.25) == 640  # 512 x 1.25
    assert oracle.capacity(8192, 8, 256, 1.0) == 256  # 256 x 1
    assert oracle.capacity(256, 8, 256, None) == 0  # no limit
    assert oracle.effective_capacity(256, 0) == 256
    assert oracle.effective_capacity(10, 40) == 10
    assert oracle.capacity(10, 1, 4, 1.0) == 3  # 2.5 rounds up


def test_capacity_double_rounding_reading():
    # READING: evaluated in IEEE double, so ((1.1 * 25) * 8) / 4 = 55.00000000000001 -> 56
    # although the exact value 1.1 * 25 * 8 / 4 is 55
    assert ((1.1 * 25) * 8) / 4 > 55
    assert oracle.capacity(25, 8, 4, 1.1) == 56


# ---------------------------------------------------------------- S3-S5 dispatch
def _all_rows(E, k):
    return list(itertools.permutations(range(E), k))


def _brute_dispatch(idx, E, C):
    """Per-expert definition: expert e keeps the first C tokens (by index) that chose it."""
    T, k = idx.shape
    Ceff = T if C <= 0 or C > T else C
    chose = {e: [t for t in range(T) if e in list(idx[t])] for e in range(E)}
    kept = {e: chose[e][:Ceff] for e in range(E)}
    off = [0]
    for e in range(E):
        off.append(off[-1] + len(kept[e]))
    dest = np.full((T, k), -1)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            if t in kept[e]:
                dest[t, j] = off[e] + kept[e].index(t)
    return [len(chose[e]) for e in range(E)], [len(kept[e]) for e in range(E)], off, dest


@pytest.mark.parametrize("k", [1, 2])
def test_dispatch_exhaustive_tiny(k):
    E, T = 3, 3
    rows = _all_rows(E, k)
    for combo in itertools.product(rows, repeat=T):
        idx = np.array(combo, dtype=np.int32)
        for C in (1, 2, 3, 0):
            tab = oracle.dispatch(idx, E, C)
            n, c, off, dest = _brute_dispatch(idx, E, C)
            assert tab["routed_counts"].tolist() == n
            assert tab["tokens_per_expert"].tolist() == c
            assert tab["expert_offsets"].tolist() == off
            assert np.array_equal(tab["dest_row"], dest)
            dropped = dest < 0
            assert tab["drops_total"] == int(dropped.sum())
            assert tab["drops_per_slot"].tolist() == dropped.sum(0).tolist()
            assert tab["fully_dropped_tokens"] == int(dropped.all(1).sum())
            for t in range(T):
                for j in range(k):
                    r = dest[t, j]
                    if r >= 0:
                        assert tab["src_token"][r] == t and tab["src_slot"][r] == j


def _random_idx(T, E, k, bias=None):
    L = rng.standard_normal((T, E)).astype(np.float32)
    if bias is not None:
        L = L + bias[None, :]
    return oracle.select_topk(L, k)


@pytest.mark.parametrize("T,E,k,C", [(500, 8, 2, 100), (300, 16, 4, 40), (257, 5, 1, 0),
                                     (400, 32, 8, 60)])
def test_dispatch_invariants_and_stable_sort(T, E, k, C):
    idx = _random_idx(T, E, k, bias=-0.7 * np.log(np.arange(1, E + 1)).astype(np.float32))
    tab = oracle.dispatch(idx, E, C)
    n, c, off = tab["routed_counts"], tab["tokens_per_expert"], tab["expert_offsets"]
    N = tab["n_kept"]
    # conservation
    assert n.sum() == T * k
    assert c.sum() == T * k - tab["drops_total"]
    assert tab["drops_per_slot"].sum() == tab["drops_total"]
    # kept rows are a bijection onto [0, N)
    dest = tab["dest_row"].reshape(-1)
    kept = dest[dest >= 0]
    assert np.array_equal(np.sort(kept), np.arange(N))
    assert np.all(tab["src_token"][N:] == -1)
    # library routine: a stable sort of the token-major list by expert, cut at C per expert
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")
    Ceff = T if C <= 0 else C
    want_src = []
    for e in range(E):
        seg = order[flat[order] == e][:Ceff]
        want_src.extend((seg // k).tolist())
    assert tab["src_token"][:N].tolist() == want_src
    # segments are token-ascending
    for e in range(E):
        s = tab["src_token"][off[e]:off[e + 1]]
        assert np.all(np.diff(s) > 0)


def test_dispatch_unlimited_keeps_everything():
    idx = _random_idx(123, 8, 2)
    tab = oracle.dispatch(idx, 8, 0)
    assert tab["drops_total"] == 0 and tab["n_kept"] == 246
    assert np.array_equal(tab["tokens_per_expert"], tab["routed_counts"])


def test_dispatch_capacity_one_keeps_first_token():
    idx = _random_idx(50, 6, 2)
    tab = oracle.dispatch(idx, 6, 1)
    for e in range(6):
        first = min(t for t in range(50) if e in idx[t])
        assert tab["src_token"][tab["expert_offsets"][e]] == first


# ---------------------------------------------------------------- S6-S8 FFN and combine
def test_dense_special_case_is_swiglu_ffn():
    # E = 1, k = 1, no capacity limit: the layer is one dense SwiGLU FFN with gate 1
    T, d, F = 9, 12, 20
    x = rng.standard_normal((T, d))
    Wr = rng.standard_normal((1, d))
    Wg, Wu, Wd = (rng.standard_normal(s) for s in ((1, F, d), (1, F, d), (1, d, F)))
    res = oracle.moe_layer(x, Wr, None, Wg, Wu, Wd, k=1, C=0)
    xt = torch.from_numpy(x)
    F_ = torch.nn.functional
    want = F_.linear(F_.silu(F_.linear(xt, torch.from_numpy(Wg[0]))) *
                     F_.linear(xt, torch.from_numpy(Wu[0])), torch.from_numpy(Wd[0])).numpy()
    assert np.max(np.abs(res["out"] - want)) < 1e-12 * np.max(np.abs(want))


def test_silu_values():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0])
    s = oracle.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(s[1] - s[2] - 1.0) < 1e-15  # silu(z) - silu(-z) = z
    assert abs(s[3] - 40.0) < 1e-12 and abs(s[4]) < 1e-15


@pytest.mark.parametrize("k,C", [(1, 0), (2, 0), (2, 20), (3, 7)])
def test_identity_experts_round_trip(k, C):
    T, d, E = 80, 16, 6
    x = rng.standard_normal((T, d)).astype(np.float32)
    L = rng.standard_normal((T, E)).astype(np.float32)
    idx = oracle.select_topk(L, k)
    w = oracle.gate_weights(L, idx)
    tab = oracle.dispatch(idx, E, C)
    xp = oracle.permute(x, tab["src_token"], tab["n_kept"])
    out = oracle.combine(xp, tab["dest_row"], w)  # identity experts: Y = X_perm
    kept_w = np.where(tab["dest_row"] >= 0, w, 0.0).sum(axis=1)
    assert np.max(np.abs(out - kept_w[:, None] * x)) < 1e-12
    if k == 1 and C == 0:
        assert np.array_equal(out.astype(np.float32), x)


def test_batched_layer_equals_rowwise_outputs():
    w = mi.WORKLOADS["tiny_f32"]
    x = mi.host_tensor_f32(w, "x")
    Wr = mi.host_tensor_f32(w, "w_router")
    Wg, Wu, Wd = (mi.host_tensor_f32(w, n) for n in ("w_gate", "w_up", "w_down"))
    C = oracle.capacity(w.T, w.k, w.E, 0.5)  # tight capacity so some rows drop
    res = oracle.moe_layer(x, Wr, None, Wg, Wu, Wd, k=w.k, C=C)
    assert res["drops_total"] > 0
    kept = res["dest_row"] >= 0
    rows = oracle.token_outputs(x, res["topk_idx"], kept, res["topk_w"],
                                lambda e: (Wg[e], Wu[e], Wd[e]))
    assert np.max(np.abs(rows - res["out"])) < 1e-12 * np.max(np.abs(res["out"]))


# ---------------------------------------------------------------- S9 statistics
def test_stats_page_example():
    rec = json.load(open(os.path.join(GOLDEN, "expert_stats_record.json")))
    n = np.array(rec["tokens_per_expert"])
    # the page's record has top_k = 2 over these counts; T is whatever gives sum n = T*k
    st = oracle.expert_stats(n, T=int(n.sum()) // 2, k=2)
    assert st["expert_max"] == rec["expert_max"]
    assert round(st["expert_max_to_mean"], 2) == rec["expert_max_to_mean"]
    assert st["dropped_tokens"] == rec["dropped_tokens"]


def test_stats_nearest_rank():
    st = oracle.expert_stats(np.arange(1, 101), T=5050, k=1)
    assert st["expert_p50"] == 50 and st["expert_p95"] == 95 and st["expert_max"] == 100


def test_streamed_expert_ffn_dense_special_case():
    # E = 1: every row is the same dense SwiGLU FFN of its token (torch F.linear), whatever
    # order src_token gathers the tokens in
    T, d, F = 11, 12, 20
    x = rng.standard_normal((T, d))
    Wg, Wu, Wd = (rng.standard_normal(s) for s in ((F, d), (F, d), (d, F)))
    src = rng.permutation(T)
    calls = []
    Y = oracle.expert_ffn_streamed(x, src, np.array([0, T]), lambda e: (calls.append(e) or
                                                                         (Wg, Wu, Wd)))
    xt = torch.from_numpy(x[src])
    F_ = torch.nn.functional
    want = F_.linear(F_.silu(F_.linear(xt, torch.from_numpy(Wg))) *
                     F_.linear(xt, torch.from_numpy(Wu)), torch.from_numpy(Wd)).numpy()
    assert calls == [0]
    assert np.max(np.abs(Y - want)) < 1e-12 * np.max(np.abs(want))


def test_streamed_layer_equals_batched_layer():
    # the streamed path (weights fetched per expert, rows gathered through src_token) and
    # the batched layer agree on a layer with drops; experts without rows are never fetched
    w = mi.WORKLOADS["tiny_f32"]
    x = mi.host_tensor_f32(w, "x")
    Wr = mi.host_tensor_f32(w, "w_router")
    Wg, Wu, Wd = (mi.host_tensor_f32(w, n) for n in ("w_gate", "w_up", "w_down"))
    C = oracle.capacity(w.T, w.k, w.E, 0.5)
    res = oracle.moe_layer(x, Wr, None, Wg, Wu, Wd, k=w.k, C=C)
    fetched = []
    Y = oracle.expert_ffn_streamed(x, res["src_token"], res["expert_offsets"],
                                   lambda e: (fetched.append(e) or (Wg[e], Wu[e], Wd[e])))
    out = oracle.combine(Y, res["dest_row"], res["topk_w"])
    assert fetched == [e for e in range(w.E) if res["tokens_per_expert"][e] > 0]
    assert np.max(np.abs(out - res["out"])) < 1e-12 * np.max(np.abs(res["out"]))


def test_streamed_layer_padded_equals_batched():
    # padded layout: the empty slots of each expert's C rows are zero rows (FFN exactly 0);
    # the streamed path skips them and equals the batched padded layer
    w = mi.WORKLOADS["tiny_f32"]
    x = mi.host_tensor_f32(w, "x")
    Wr = mi.host_tensor_f32(w, "w_router")
    Wg, Wu, Wd = (mi.host_tensor_f32(w, n) for n in ("w_gate", "w_up", "w_down"))
    res = oracle.moe_layer(x, Wr, None, Wg, Wu, Wd, k=w.k, C=24, pad_to_capacity=True)
    assert np.any(res["src_token"] < 0)
    Y = oracle.expert_ffn_streamed(x, res["src_token"], res["expert_offsets"],
                                   lambda e: (Wg[e], Wu[e], Wd[e]))
    assert np.array_equal(Y[res["src_token"] < 0], np.zeros_like(Y[res["src_token"] < 0]))
    assert np.max(np.abs(Y - res["y_perm"])) < 1e-12 * np.max(np.abs(res["y_perm"]))
