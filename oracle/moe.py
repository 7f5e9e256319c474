"""CPU oracle for one GPU's share of a Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg may import or call this module; the library's product path never does, and this module
imports nothing from it.  It is plain numpy in float64, written from the pages' description
of the layer, slow on purpose and meant to be checked by eye.

Pages cited (title, then the section a step follows):
  [EP-serving]  aiunderstanding.org, "Expert parallelism for MoE serving" (Russian, Wolof and
                Indonesian versions of one article).
  [EP-checks]   airouter.kz blog, "Expert parallelism in MoE needs measurements before
                launch" ("Экспертный параллелизм MoE требует замеров до запуска").
Steps the pages leave open are marked READING; they follow the layer's specification
(softmax top-k with lowest-index tie-break and renormalised gates, a SwiGLU expert FFN,
capacity-factor truncation with dropped-token accounting) in its plainest form.

Parity unpinned: the nearest-rank reading of expert_p50 / expert_p95 in expert_stats()
(the page's printed example matches no standard percentile rule, so nothing pins it).
"""
from __future__ import annotations

import math
from typing import Callable, Optional

import numpy as np


# ------------------------------------------------------------------------------------------
# S1  router logits
# ------------------------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_router: np.ndarray,
                  b_router: Optional[np.ndarray] = None) -> np.ndarray:
    """L[t, e] = sum_i x[t, i] * w_router[e, i] + b_router[e], accumulated in float64 and
    stored as float32.

    [EP-serving] "Deep dive": a router scores the experts for each token.  READING: the
    score is a linear map of the token (weights [E, d], nn.Linear layout) plus an optional
    per-expert bias, and the logits are kept in fp32, the precision both sides route from.
    """
    L = np.asarray(x, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64).T
    if b_router is not None:
        L = L + np.asarray(b_router, dtype=np.float64)[None, :]
    return L.astype(np.float32)


# ------------------------------------------------------------------------------------------
# S2  top-k selection and gates
# ------------------------------------------------------------------------------------------
def select_topk(logits: np.ndarray, k: int, n_groups: int = 1,
                topk_groups: Optional[int] = None) -> np.ndarray:
    """idx[t, j] = the (j+1)-th best expert of token t.

    [EP-serving] "Deep dive": the router picks the top-k experts (often 1 or 2) per token.
    READING: "best" is the order (logit descending, expert index ascending), so equal logits
    go to the lower index; -0.0 and +0.0 are equal.  Softmax is strictly increasing, so this
    is the top-k of the softmax probabilities as well.  A stable sort of the negated logits
    is exactly that order.

    Group-limited selection ([EP-checks] "Routing is a system-level decision": routing that
    limits how many nodes a token may reach shapes the exchange).  The pages fix neither
    the group count nor the limit, so both are parameters.  READING: the E experts form
    n_groups groups of E / n_groups consecutive indices; a group's score is its best logit;
    a token keeps the topk_groups groups of highest score (ties to the lower group index)
    and picks its k experts among theirs in the order above.
    """
    L = np.asarray(logits, dtype=np.float32)
    assert np.all(np.isfinite(L)), "non-finite logits are outside the oracle's contract"
    T, E = L.shape
    assert 1 <= k <= E
    canon = L + np.float32(0.0)  # -0.0 + 0.0 == +0.0
    if n_groups > 1 and topk_groups is not None and topk_groups < n_groups:
        assert E % n_groups == 0 and 1 <= topk_groups
        gs = E // n_groups
        assert k <= topk_groups * gs
        score = canon.reshape(T, n_groups, gs).max(axis=2)
        chosen = np.argsort(-score, axis=1, kind="stable")[:, :topk_groups]
        allowed = np.zeros((T, n_groups), dtype=bool)
        np.put_along_axis(allowed, chosen, True, axis=1)
        canon = np.where(np.repeat(allowed, gs, axis=1), canon.astype(np.float64), -np.inf)
    order = np.argsort(-canon, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def selection_logits(logits: np.ndarray, b_router: Optional[np.ndarray]) -> np.ndarray:
    """Logits that decide the selection when the bias shifts the selection only: the fp32
    sum L + b, rounded to fp32 like every logit the selection sees.

    [EP-serving] "Deep dive" (the router's choice decides which experts run) with
    [EP-checks] "Routing is a system-level decision" (balancing the load is part of
    routing).  READING: with a selection-only bias (the auxiliary-loss-free balancing
    style) the bias moves which experts are chosen but the gates come from the unbiased
    logits.
    """
    L = np.asarray(logits, dtype=np.float32)
    if b_router is None:
        return L
    return (L + np.asarray(b_router, dtype=np.float32)[None, :]).astype(np.float32)


def gate_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """w[t, j] = exp(L[t, idx[t, j]] - m) / sum_i exp(L[t, idx[t, i]] - m), m = best logit.

    READING (the layer's specification): softmax over all experts, restricted to the
    selected ones and renormalised to sum 1.  The full-softmax denominator cancels, so only
    the selected logits are needed.
    """
    L = np.asarray(logits, dtype=np.float64)
    sel = np.take_along_axis(L, np.asarray(idx, dtype=np.int64), axis=1)
    m = sel.max(axis=1, keepdims=True)
    p = np.exp(sel - m)
    return p / p.sum(axis=1, keepdims=True)


# ------------------------------------------------------------------------------------------
# S4  capacity
# ------------------------------------------------------------------------------------------
def capacity(T: int, k: int, E: int, cf: Optional[float]) -> int:
    """Per-expert capacity C; 0 means no limit.

    [EP-checks] "Capacity factor changes quality, memory and tail latency": capacity is the
    mean number of tokens per expert times the capacity factor, rounding left to the engine;
    a disabled limit means effectively unlimited capacity.  [EP-checks] "Mean expert load
    proves almost nothing" gives the mean as sum_e n_e / E = T*k / E.
    READING: C = ceil(((cf * T) * k) / E) evaluated in IEEE double; cf None or <= 0 is
    'no limit'.
    """
    if cf is None or not (cf > 0):
        return 0
    return int(math.ceil(((float(cf) * T) * k) / E))


def effective_capacity(T: int, C: int) -> int:
    """No expert can receive more than T rows, so 'no limit' and C > T both mean C = T."""
    return T if (C <= 0 or C > T) else C


# ------------------------------------------------------------------------------------------
# S3-S5  dispatch: counts, capacity truncation, offsets, permutation
# ------------------------------------------------------------------------------------------
def dispatch(idx: np.ndarray, E: int, C: int, slot_major: bool = False,
             pad_to_capacity: bool = False) -> dict:
    """Routing tables for the single-GPU stand-in of the dispatch all-to-all.

    [EP-serving] "Technical details": tokens are sent to their experts, experts get
    capacity-limited buffers and overflow tokens are dropped.  [EP-checks] "Capacity factor
    changes quality, memory and tail latency": in capacity mode overflow is dropped before
    the exchange, so every keep/drop decision here is made before any row moves.
    READING (drop priority, not on the pages): first come, first kept.  Assignments are
    visited in token-major order (t, j) by default, or slot-major order (j, t) -- every
    first choice before any second choice -- when slot_major; the assignment (t, j) -> e
    has position pos = number of assignments to e visited before it, and it is kept iff
    pos < C.  Kept rows of an expert are stored in visit order.

    Buffers: packed (default), expert e's rows are [off_e, off_{e+1}) with off the exclusive
    scan of the kept counts; with pad_to_capacity every expert owns C slots, rows
    [e * C, (e + 1) * C), and the slots past its kept count stay empty (src_token -1, zero
    rows).  [EP-serving] "Technical details" (fixed-capacity expert buffers keep the GEMM
    shapes regular) and [EP-checks] "Capacity factor changes quality, memory and tail
    latency" (padding to capacity spends memory and compute on empty slots).

    Returns routed_counts n_e, tokens_per_expert c_e = min(n_e, C), expert_offsets [E+1],
    pos, dest_row [T, k] (-1 when dropped), src_token / src_slot over the row slots (-1
    where no row), n_kept N = sum c_e, n_rows (row slots: T*k packed, E*C padded), and drops
    (total, per slot, tokens with every slot dropped).
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    Ceff = effective_capacity(T, C)
    pos = np.empty((T, k), dtype=np.int64)
    seen = [0] * E
    walk = ([(t, j) for j in range(k) for t in range(T)] if slot_major
            else [(t, j) for t in range(T) for j in range(k)])
    for t, j in walk:
        e = int(idx[t, j])
        pos[t, j] = seen[e]
        seen[e] += 1
    routed = np.array(seen, dtype=np.int64)
    kept_counts = np.minimum(routed, Ceff)
    if pad_to_capacity:
        offsets = np.arange(E + 1, dtype=np.int64) * Ceff
        n_rows = E * Ceff
    else:
        offsets = np.zeros(E + 1, dtype=np.int64)
        offsets[1:] = np.cumsum(kept_counts)
        n_rows = T * k
    kept = pos < Ceff
    dest = np.where(kept, offsets[idx] + pos, -1)
    src_token = np.full(n_rows, -1, dtype=np.int64)
    src_slot = np.full(n_rows, -1, dtype=np.int64)
    for t, j in zip(*np.nonzero(kept)):
        src_token[dest[t, j]] = t
        src_slot[dest[t, j]] = j
    dropped = ~kept
    return {
        "routed_counts": routed,
        "tokens_per_expert": kept_counts,
        "expert_offsets": offsets,
        "capacity": Ceff,
        "pos": pos,
        "dest_row": dest,
        "src_token": src_token,
        "src_slot": src_slot,
        "n_kept": int(kept_counts.sum()),
        "n_rows": int(n_rows),
        "drops_total": int(dropped.sum()),
        "drops_per_slot": dropped.sum(axis=0).astype(np.int64),
        "fully_dropped_tokens": int(dropped.all(axis=1).sum()),
    }


def permute(x: np.ndarray, src_token: np.ndarray, n_rows: int) -> np.ndarray:
    """X_perm[r] = x[src_token[r]] for the first n_rows row slots, a zero row where
    src_token[r] = -1 (the pack step of [EP-checks] "All-to-all must be profiled separately
    from compute")."""
    x = np.asarray(x)
    src = np.asarray(src_token[:n_rows], dtype=np.int64)
    out = np.zeros((n_rows, x.shape[1]), dtype=x.dtype)
    has = src >= 0
    out[has] = x[src[has]]
    return out


# ------------------------------------------------------------------------------------------
# S6-S7  expert FFN
# ------------------------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(rows: np.ndarray, w_gate_e: np.ndarray, w_up_e: np.ndarray,
               w_down_e: np.ndarray) -> np.ndarray:
    """One expert on a block of rows: silu(r Wg^T) * (r Wu^T), then times Wd^T, in float64.

    [EP-serving] "Deep dive": each expert is a small feed-forward network.  READING (the
    layer's specification): the SwiGLU form, weights in nn.Linear layout
    (Wg, Wu: [F, d]; Wd: [d, F]).
    """
    r = np.asarray(rows, dtype=np.float64)
    g = r @ np.asarray(w_gate_e, dtype=np.float64).T
    u = r @ np.asarray(w_up_e, dtype=np.float64).T
    h = silu(g) * u
    return h @ np.asarray(w_down_e, dtype=np.float64).T


def expert_ffn(x_perm: np.ndarray, expert_offsets: np.ndarray, w_gate, w_up, w_down
               ) -> np.ndarray:
    """Y[r] = FFN_e(X_perm[r]) for each expert's segment [off_e, off_{e+1})."""
    off = np.asarray(expert_offsets, dtype=np.int64)
    E = off.shape[0] - 1
    N = int(off[E])
    d = np.asarray(x_perm).shape[1]
    Y = np.zeros((N, d), dtype=np.float64)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            Y[a:b] = swiglu_ffn(x_perm[a:b], w_gate[e], w_up[e], w_down[e])
    return Y


def expert_ffn_streamed(x: np.ndarray, src_token: np.ndarray, expert_offsets: np.ndarray,
                        expert_weights: Callable[[int], tuple],
                        progress: Optional[Callable[[int], None]] = None) -> np.ndarray:
    """expert_ffn(permute(x, src_token, N), expert_offsets, ...) for layers whose weights are
    too large to hold at once: Y[r] = FFN_e(x[src_token[r]]) for the rows r of each expert's
    segment [off_e, off_{e+1}), with expert_weights(e) -> (Wg_e, Wu_e, Wd_e) called only for
    experts that hold rows, one expert at a time.  Same steps as expert_ffn, in the same
    expert order; progress(e), if given, is called after each expert.  An empty slot of the
    padded layout (src_token -1) is a zero row, whose FFN is exactly zero (silu(0) * 0 = 0),
    so its Y row stays zero."""
    off = np.asarray(expert_offsets, dtype=np.int64)
    src = np.asarray(src_token, dtype=np.int64)
    E = off.shape[0] - 1
    N = int(off[E])
    Y = np.zeros((N, np.asarray(x).shape[1]), dtype=np.float64)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        rows = src[a:b]
        has = np.nonzero(rows >= 0)[0]
        if has.size:
            wg, wu, wd = expert_weights(e)
            Y[a + has] = swiglu_ffn(np.asarray(x)[rows[has]], wg, wu, wd)
        if progress is not None:
            progress(e)
    return Y


# ------------------------------------------------------------------------------------------
# S8  combine
# ------------------------------------------------------------------------------------------
def combine(y_perm: np.ndarray, dest_row: np.ndarray, gates: np.ndarray) -> np.ndarray:
    """out[t] = sum over slots j with dest_row[t, j] >= 0 of gates[t, j] * Y[dest_row[t, j]].

    [EP-serving] "Technical details": the combine step brings the expert outputs back to
    their tokens.  READING: the gates of dropped assignments are not renormalised, and a
    token with every slot dropped gets a zero row.
    """
    dest = np.asarray(dest_row, dtype=np.int64)
    w = np.asarray(gates, dtype=np.float64)
    T, k = dest.shape
    Y = np.asarray(y_perm, dtype=np.float64)
    out = np.zeros((T, Y.shape[1]), dtype=np.float64)
    for j in range(k):
        m = dest[:, j] >= 0
        out[m] += w[m, j][:, None] * Y[dest[m, j]]
    return out


# ------------------------------------------------------------------------------------------
# S9  per-layer expert statistics
# ------------------------------------------------------------------------------------------
def expert_stats(routed_counts: np.ndarray, T: int, k: int,
                 tokens_per_expert: Optional[np.ndarray] = None,
                 dropped: int = 0) -> dict:
    """The per-layer record of [EP-checks] "Mean expert load proves almost nothing".

    n_e = assignments to expert e after top-k, mean mu = sum_e n_e / E, expert_max and
    expert_max_to_mean = max / mu.  READING: the statistics are over routed counts (before
    capacity truncation); p50 / p95 use the nearest rank, s[ceil(q * E) - 1] of the sorted
    counts (parity unpinned).
    """
    n = np.asarray(routed_counts, dtype=np.int64)
    E = n.shape[0]
    mu = n.sum() / E
    s = np.sort(n)

    def nearest_rank(q):
        return int(s[max(0, math.ceil(q * E) - 1)])

    rec = {
        "active_tokens": int(T),
        "top_k": int(k),
        "routed_per_expert": n.tolist(),
        "expert_p50": nearest_rank(0.50),
        "expert_p95": nearest_rank(0.95),
        "expert_max": int(s[-1]),
        "expert_mean": float(mu),
        "expert_max_to_mean": float(s[-1] / mu) if mu > 0 else float("nan"),
        "dropped_tokens": int(dropped),
    }
    if tokens_per_expert is not None:
        rec["tokens_per_expert"] = np.asarray(tokens_per_expert, dtype=np.int64).tolist()
    return rec


def routing_record(idx: np.ndarray, dest_row: np.ndarray, E: int,
                   placement: Optional[np.ndarray] = None,
                   ranks_per_node: Optional[int] = None) -> dict:
    """Observability record of one layer's routing beyond the expert counts.

    [EP-checks] "Mean expert load proves almost nothing" (the share held by the busiest
    experts, the distribution of the second choice), "Capacity factor changes quality,
    memory and tail latency" (which choices get dropped) and "Routing is a system-level
    decision" (load per GPU and per node under a given expert placement).  READINGS:
      routed_by_slot[j][e] = assignments of slot j to expert e; kept_by_slot likewise for
        kept ones;
      top_5_percent_expert_share = routed assignments of the ceil(0.05 E) busiest experts
        over all routed assignments;
      slot_max_to_mean[j] = max_e routed_by_slot[j][e] / (T / E), the imbalance of the
        (j+1)-th choice alone;
      drop_share_per_slot[j] = dropped assignments of slot j over all dropped (0 when
        nothing is dropped);
      with placement[e] = the rank holding expert e: rank_load[r] = assignments routed to
        rank r's experts, node_load[n] = sum over ranks n * ranks_per_node ... + ranks_per_node
        - 1, each with its max / mean.
    """
    idx = np.asarray(idx, dtype=np.int64)
    dest = np.asarray(dest_row, dtype=np.int64)
    T, k = idx.shape
    routed_by_slot = np.zeros((k, E), dtype=np.int64)
    kept_by_slot = np.zeros((k, E), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            routed_by_slot[j, idx[t, j]] += 1
            if dest[t, j] >= 0:
                kept_by_slot[j, idx[t, j]] += 1
    n = routed_by_slot.sum(axis=0)
    top = int(math.ceil(0.05 * E))
    busiest = np.sort(n)[::-1][:top]
    total = int(n.sum())
    dropped_by_slot = routed_by_slot.sum(axis=1) - kept_by_slot.sum(axis=1)
    dropped = int(dropped_by_slot.sum())
    rec = {
        "routed_by_slot": routed_by_slot.tolist(),
        "kept_by_slot": kept_by_slot.tolist(),
        "top_5_percent_experts": top,
        "top_5_percent_expert_share": float(busiest.sum() / total) if total else 0.0,
        "slot_max_to_mean": [float(routed_by_slot[j].max() / (T / E)) if T else 0.0
                             for j in range(k)],
        "drop_share_per_slot": [float(dropped_by_slot[j] / dropped) if dropped else 0.0
                                for j in range(k)],
    }
    if placement is not None:
        pl = np.asarray(placement, dtype=np.int64)
        n_ranks = int(pl.max()) + 1
        rank_load = np.zeros(n_ranks, dtype=np.int64)
        for e in range(E):
            rank_load[pl[e]] += n[e]
        rec["rank_load"] = rank_load.tolist()
        rec["rank_max_to_mean"] = float(rank_load.max() / rank_load.mean()) if total else 0.0
        if ranks_per_node:
            n_nodes = (n_ranks + ranks_per_node - 1) // ranks_per_node
            node_load = np.zeros(n_nodes, dtype=np.int64)
            for r in range(n_ranks):
                node_load[r // ranks_per_node] += rank_load[r]
            rec["node_load"] = node_load.tolist()
            rec["node_max_to_mean"] = float(node_load.max() / node_load.mean()) if total else 0.0
    return rec


# ------------------------------------------------------------------------------------------
# the whole layer
# ------------------------------------------------------------------------------------------
def moe_layer(x, w_router, b_router, w_gate, w_up, w_down, k: int, C: int,
              logits: Optional[np.ndarray] = None, bias_selection_only: bool = False,
              n_groups: int = 1, topk_groups: Optional[int] = None,
              slot_major: bool = False, pad_to_capacity: bool = False) -> dict:
    """Router -> dispatch -> expert FFN -> combine on one GPU's share (expert parallel size
    1: every expert is local and no all-to-all runs, the control run of [EP-checks]
    "All-to-all must be profiled separately from compute").

    If `logits` is given the oracle routes from it instead of computing S1 (with
    bias_selection_only these are the unbiased logits and b_router still shifts the
    selection).
    """
    if logits is None:
        logits = router_logits(x, w_router, None if bias_selection_only else b_router)
    E = logits.shape[1]
    sel = selection_logits(logits, b_router) if bias_selection_only else logits
    idx = select_topk(sel, k, n_groups, topk_groups)
    gates = gate_weights(logits, idx)
    tab = dispatch(idx, E, C, slot_major=slot_major, pad_to_capacity=pad_to_capacity)
    n_rows = tab["n_rows"] if pad_to_capacity else tab["n_kept"]
    xp = permute(x, tab["src_token"], n_rows)
    Y = expert_ffn(xp, tab["expert_offsets"], w_gate, w_up, w_down)
    out = combine(Y, tab["dest_row"], gates)
    res = dict(tab)
    res.update(logits=logits, topk_idx=idx, topk_w=gates, x_perm=xp, y_perm=Y, out=out)
    return res


def token_outputs(x_rows: np.ndarray, idx_rows: np.ndarray, kept_rows: np.ndarray,
                  gates_rows: np.ndarray,
                  expert_weights: Callable[[int], tuple]) -> np.ndarray:
    """out for a sample of tokens, one token at a time, for layers too large to hold.

    Row-wise identity of the layer: Y[dest[t, j]] = FFN_{idx[t, j]}(x[t]), so out[t] needs
    only token t, its routing row and the weights of its kept experts.
    expert_weights(e) returns (Wg_e, Wu_e, Wd_e).
    """
    xs = np.asarray(x_rows, dtype=np.float64)
    n, k = np.asarray(idx_rows).shape
    y = {}
    need = sorted({int(e) for e, kp in zip(np.ravel(idx_rows), np.ravel(kept_rows)) if kp})
    for e in need:  # one expert's weights at a time
        wg, wu, wd = expert_weights(e)
        for t in range(n):
            for j in range(k):
                if kept_rows[t, j] and int(idx_rows[t, j]) == e:
                    y[(t, j)] = swiglu_ffn(xs[t:t + 1], wg, wu, wd)[0]
    out = np.zeros_like(xs)
    for t in range(n):
        for j in range(k):  # slot order, as in combine()
            if kept_rows[t, j]:
                out[t] += float(gates_rows[t, j]) * y[(t, j)]
    return out
