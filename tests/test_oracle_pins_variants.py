"""Pins of the oracle's routing and dispatch variants to facts outside itself.

Variants: group-limited top-k, a router bias that shifts the selection only, slot-major drop
priority, pad-to-capacity buffers, and the routing observability record.  Each is pinned by
brute force over tiny inputs, a special case that reduces to the default path or to a
library routine, or an invariant between tables computed two ways.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle

rng = np.random.default_rng(4321)


# ---------------------------------------------------------------- group-limited top-k
def _better(row, a, b):
    return row[a] > row[b] or (row[a] == row[b] and a < b)


def _brute_group_topk(row, k, n_groups, m):
    """Groups: the m-subset whose every member beats every outsider under (best value desc,
    group index asc); then the k experts of those groups that beat every other candidate."""
    E = len(row)
    gs = E // n_groups
    score = [max(float(row[e]) + 0.0 for e in range(g * gs, (g + 1) * gs)) for g in range(n_groups)]

    def gbetter(a, b):
        return score[a] > score[b] or (score[a] == score[b] and a < b)

    subsets = [S for S in itertools.combinations(range(n_groups), m)
               if all(gbetter(s, o) for s in S for o in range(n_groups) if o not in S)]
    assert len(subsets) == 1
    cand = [e for g in subsets[0] for e in range(g * gs, (g + 1) * gs)]
    r = [float(v) + 0.0 for v in row]
    out = []
    while len(out) < k:
        rest = [c for c in cand if c not in out]
        top = [c for c in rest if all(_better(r, c, o) for o in rest if o != c)]
        assert len(top) == 1
        out.append(top[0])
    return out


def test_group_topk_brute_force_tie_grid():
    vals = np.array([-1.0, -0.0, 0.0, 1.0], dtype=np.float32)
    rows = np.array(list(itertools.product(vals, repeat=4)), dtype=np.float32)
    for k in (1, 2):
        got = oracle.select_topk(rows, k, n_groups=2, topk_groups=1)
        for t in range(rows.shape[0]):
            assert list(got[t]) == _brute_group_topk(rows[t], k, 2, 1), (rows[t], k)


@pytest.mark.parametrize("E,G,M", [(6, 3, 2), (8, 4, 2), (8, 4, 3), (9, 3, 1)])
def test_group_topk_brute_force_random(E, G, M):
    L = rng.integers(-2, 3, size=(200, E)).astype(np.float32)
    gs = E // G
    for k in range(1, M * gs + 1):
        got = oracle.select_topk(L, k, n_groups=G, topk_groups=M)
        for t in range(L.shape[0]):
            assert list(got[t]) == _brute_group_topk(L[t], k, G, M)


def test_group_topk_special_cases_are_plain_topk():
    L = rng.standard_normal((300, 16)).astype(np.float32)
    for k in (1, 3, 8):
        plain = oracle.select_topk(L, k)
        assert np.array_equal(oracle.select_topk(L, k, n_groups=1, topk_groups=1), plain)
        assert np.array_equal(oracle.select_topk(L, k, n_groups=4, topk_groups=4), plain)


def test_group_topk_stays_in_chosen_groups():
    E, G, M, k = 64, 8, 3, 6
    L = rng.standard_normal((500, E)).astype(np.float32)
    idx = oracle.select_topk(L, k, n_groups=G, topk_groups=M)
    gs = E // G
    score = L.reshape(-1, G, gs).max(axis=2)
    for t in range(L.shape[0]):
        groups = set((idx[t] // gs).tolist())
        assert len(groups) <= M
        # no group outside the selection has a strictly better score than one inside
        worst_in = min(score[t, g] for g in groups)
        assert all(score[t, g] <= worst_in for g in range(G) if g not in groups)


# ---------------------------------------------------------------- selection-only bias
def test_selection_bias_zero_is_plain_routing():
    L = rng.standard_normal((100, 8)).astype(np.float32)
    sel = oracle.selection_logits(L, np.zeros(8, dtype=np.float32))
    assert np.array_equal(sel, L)


def test_selection_bias_moves_choice_not_gates():
    T, E, k = 200, 8, 2
    L = rng.standard_normal((T, E)).astype(np.float32)
    b = np.zeros(E, dtype=np.float32)
    b[3] = 100.0  # larger than any logit gap: expert 3 is always the first choice
    idx = oracle.select_topk(oracle.selection_logits(L, b), k)
    assert np.all(idx[:, 0] == 3)
    w = oracle.gate_weights(L, idx)
    # library: softmax over the selected *unbiased* logits
    sel = np.take_along_axis(L.astype(np.float64), idx.astype(np.int64), axis=1)
    want = torch.softmax(torch.from_numpy(sel), dim=1).numpy()
    assert np.max(np.abs(w - want)) < 1e-15


def test_selection_bias_k_equals_E_gates_are_softmax():
    T, E = 50, 6
    L = rng.standard_normal((T, E)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    idx = oracle.select_topk(oracle.selection_logits(L, b), E)
    w = oracle.gate_weights(L, idx)
    full = torch.softmax(torch.from_numpy(L.astype(np.float64)), dim=1).numpy()
    assert np.max(np.abs(w - np.take_along_axis(full, idx.astype(np.int64), axis=1))) < 1e-15


def test_selection_logits_are_fp32_sums():
    L = np.array([[1.0, 2.0**-30]], dtype=np.float32)
    b = np.array([2.0**-30, 1.0], dtype=np.float32)
    sel = oracle.selection_logits(L, b)
    assert sel.dtype == np.float32
    # in fp32 both sums round to 1.0 exactly: a tie, broken to the lower index
    assert sel[0, 0] == sel[0, 1] == np.float32(1.0)
    assert oracle.select_topk(sel, 1)[0, 0] == 0


# ---------------------------------------------------------------- slot-major drop priority
def _brute_slot_major(idx, E, C):
    """Expert e keeps the first C of: its first-choice tokens in index order, then its
    second-choice tokens in index order, and so on."""
    T, k = idx.shape
    Ceff = T if C <= 0 or C > T else C
    queue = {e: [(t, j) for j in range(k) for t in range(T) if idx[t, j] == e] for e in range(E)}
    kept = {e: queue[e][:Ceff] for e in range(E)}
    off = [0]
    for e in range(E):
        off.append(off[-1] + len(kept[e]))
    dest = np.full((T, k), -1)
    for e in range(E):
        for p, (t, j) in enumerate(kept[e]):
            dest[t, j] = off[e] + p
    return [len(kept[e]) for e in range(E)], off, dest


@pytest.mark.parametrize("k", [1, 2])
def test_slot_major_exhaustive_tiny(k):
    E, T = 3, 3
    rows = [list(p) for p in itertools.permutations(range(E), k)]
    for combo in itertools.product(rows, repeat=T):
        idx = np.array(combo, dtype=np.int32)
        for C in (1, 2, 0):
            tab = oracle.dispatch(idx, E, C, slot_major=True)
            c, off, dest = _brute_slot_major(idx, E, C)
            assert tab["tokens_per_expert"].tolist() == c
            assert tab["expert_offsets"].tolist() == off
            assert np.array_equal(tab["dest_row"], dest)


@pytest.mark.parametrize("T,E,k,C", [(500, 8, 2, 100), (300, 16, 4, 40), (400, 32, 8, 60)])
def test_slot_major_is_stable_sort_of_slot_major_list(T, E, k, C):
    L = rng.standard_normal((T, E)).astype(np.float32) - 0.7 * np.log(np.arange(1, E + 1))
    idx = oracle.select_topk(L.astype(np.float32), k)
    tab = oracle.dispatch(idx, E, C, slot_major=True)
    flat = idx.T.reshape(-1)  # p = j * T + t
    order = np.argsort(flat, kind="stable")
    want_src, want_slot = [], []
    for e in range(E):
        seg = order[flat[order] == e][:C]
        want_src += (seg % T).tolist()
        want_slot += (seg // T).tolist()
    N = tab["n_kept"]
    assert tab["src_token"][:N].tolist() == want_src
    assert tab["src_slot"][:N].tolist() == want_slot
    # first choices are dropped only beyond C first choices of one expert
    n0 = np.bincount(idx[:, 0], minlength=E)
    assert tab["drops_per_slot"][0] == int(np.maximum(n0 - C, 0).sum())
    # routed counts and kept counts do not depend on the order
    tm = oracle.dispatch(idx, E, C)
    assert np.array_equal(tab["routed_counts"], tm["routed_counts"])
    assert np.array_equal(tab["tokens_per_expert"], tm["tokens_per_expert"])
    assert tab["drops_total"] == tm["drops_total"]


def test_slot_major_k1_is_token_major():
    idx = oracle.select_topk(rng.standard_normal((300, 8)).astype(np.float32), 1)
    a, b = oracle.dispatch(idx, 8, 20), oracle.dispatch(idx, 8, 20, slot_major=True)
    for key in ("dest_row", "src_token", "expert_offsets"):
        assert np.array_equal(a[key], b[key])


# ---------------------------------------------------------------- pad-to-capacity buffers
@pytest.mark.parametrize("slot_major", [False, True])
def test_pad_tables_relate_to_packed(slot_major):
    T, E, k, C = 300, 8, 2, 60
    idx = oracle.select_topk(rng.standard_normal((T, E)).astype(np.float32), k)
    pk = oracle.dispatch(idx, E, C, slot_major=slot_major)
    pd = oracle.dispatch(idx, E, C, slot_major=slot_major, pad_to_capacity=True)
    assert pd["n_rows"] == E * C and pd["expert_offsets"].tolist() == list(range(0, E * C + 1, C))
    e = idx.astype(np.int64)
    kept = pk["dest_row"] >= 0
    want = np.where(kept, e * C + (pk["dest_row"] - pk["expert_offsets"][e]), -1)
    assert np.array_equal(pd["dest_row"], want)
    assert int((pd["src_token"] >= 0).sum()) == pk["n_kept"]
    for ee in range(E):
        seg = pd["src_token"][ee * C:(ee + 1) * C]
        c = pk["tokens_per_expert"][ee]
        assert np.array_equal(seg[:c], pk["src_token"][pk["expert_offsets"][ee]:pk["expert_offsets"][ee + 1]])
        assert np.all(seg[c:] == -1)


def test_pad_layer_equals_packed_layer():
    T, d, E, k, F, C = 60, 16, 6, 2, 24, 14
    x = rng.standard_normal((T, d))
    Wr = rng.standard_normal((E, d))
    Wg, Wu, Wd = (rng.standard_normal(s) for s in ((E, F, d), (E, F, d), (E, d, F)))
    a = oracle.moe_layer(x, Wr, None, Wg, Wu, Wd, k=k, C=C)
    b = oracle.moe_layer(x, Wr, None, Wg, Wu, Wd, k=k, C=C, pad_to_capacity=True)
    assert a["drops_total"] > 0
    assert np.array_equal(a["out"], b["out"])
    empty = b["src_token"] < 0
    assert np.all(b["x_perm"][empty] == 0) and np.all(b["y_perm"][empty] == 0)


# ---------------------------------------------------------------- observability record
def test_record_top5_share_closed_forms():
    E, k = 40, 1
    T = 400
    idx = np.repeat(np.arange(E), T // E)[:, None]  # every expert gets T / E tokens
    rec = oracle.routing_record(idx, np.zeros_like(idx), E)
    assert rec["top_5_percent_experts"] == 2
    assert rec["top_5_percent_expert_share"] == pytest.approx(2 / 40, abs=0)
    hot = np.zeros((T, 1), dtype=np.int64)  # everything on expert 0
    assert oracle.routing_record(hot, np.zeros_like(hot), E)["top_5_percent_expert_share"] == 1.0
    assert math.ceil(0.05 * 256) == oracle.routing_record(hot, hot, 256)["top_5_percent_experts"]


@pytest.mark.parametrize("slot_major", [False, True])
def test_record_consistent_with_dispatch(slot_major):
    T, E, k, C = 400, 16, 4, 90
    L = rng.standard_normal((T, E)).astype(np.float32) - 0.5 * np.log(np.arange(1, E + 1))
    idx = oracle.select_topk(L.astype(np.float32), k)
    tab = oracle.dispatch(idx, E, C, slot_major=slot_major)
    placement = np.arange(E) // 2  # 8 ranks of 2 experts, 2 ranks per node
    rec = oracle.routing_record(idx, tab["dest_row"], E, placement, ranks_per_node=2)
    rbs, kbs = np.array(rec["routed_by_slot"]), np.array(rec["kept_by_slot"])
    assert np.all(rbs.sum(axis=1) == T)
    assert np.array_equal(rbs.sum(axis=0), tab["routed_counts"])
    assert np.array_equal(kbs.sum(axis=0), tab["tokens_per_expert"])
    drops = tab["drops_per_slot"]
    assert tab["drops_total"] > 0
    assert rec["drop_share_per_slot"] == pytest.approx((drops / drops.sum()).tolist())
    assert rec["rank_load"] == (tab["routed_counts"][0::2] + tab["routed_counts"][1::2]).tolist()
    assert sum(rec["node_load"]) == T * k and len(rec["node_load"]) == 4
    st = oracle.expert_stats(rbs[0], T=T, k=1)
    assert rec["slot_max_to_mean"][0] == pytest.approx(st["expert_max_to_mean"])
