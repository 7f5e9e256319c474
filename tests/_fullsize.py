"""Every-token parity of one full-size moe_layer call against the oracle.

The oracle routes from the GPU's own fp32 logits (which are first checked against its
float64 logits of the seeded inputs), so every routing table must match bit for bit; then
it computes every kept row with each expert's weights regenerated from the seeded generator
one expert at a time (the DeepSeek-V3-shaped layers hold 22.5 GB of weights), combines them
in slot order and compares all T output rows with the layer's.
"""
from __future__ import annotations

import time

import numpy as np

import moe_inputs as mi
import oracle
import routing_expert_ffn_router_amd as moe
from _util import OUT_TOL, device_inputs, log, logits_tol, near_tie_ok, rel_err, to_host


def expert_weights(w):
    """e -> (Wg_e, Wu_e, Wd_e) of workload w, regenerated on the host (float32, exact)."""
    def get(e):
        return tuple(mi.host_tensor_f32(w, n, e, 1)[0] for n in ("w_gate", "w_up", "w_down"))
    return get


def check_layer_every_token(w, s, torch):
    """Run moe_layer on shape s of workload w and compare it with the oracle everywhere."""
    flags = s.flags
    sel_only = bool(flags & moe.MOE_FLAG_BIAS_SELECTION_ONLY)
    G, M = (s.n_groups, s.topk_groups) if s.n_groups > 1 else (1, None)
    dev = device_inputs(w)
    lay = moe.MoELayer(s)
    lay(dev["x"], dev["w_router"], dev["b_router"], dev["w_gate"], dev["w_up"], dev["w_down"])
    torch.cuda.synchronize()
    del dev
    torch.cuda.empty_cache()
    assert lay.status.item() == 0

    # S1: the GPU's logits against the oracle's float64 logits of the same inputs
    b = mi.router_bias(w)
    x = mi.host_tensor_f32(w, "x")
    L_ref = oracle.router_logits(x, mi.host_tensor_f32(w, "w_router"), None if sel_only else b)
    L_gpu = lay.view("logits").cpu().numpy()
    tol = logits_tol(L_ref)
    dl = float(np.max(np.abs(L_gpu - L_ref)))
    log(f"  max|dL| {dl:.3e} (tol {tol:.3e})")
    assert dl <= tol
    idx_gpu = lay.view("topk_idx").cpu().numpy()
    # S1 -> S2: where the GPU's selection differs from the oracle's own routing, the logits
    # of the swapped experts are within the logits tolerance (near-ties)
    ref_sel = oracle.selection_logits(L_ref, b) if sel_only else L_ref
    bad, unexplained = near_tie_ok(ref_sel, idx_gpu, oracle.select_topk(ref_sel, w.k, G, M),
                                   tol)
    log(f"  selection from float64 logits differs on {len(bad)} tokens (near-ties)")
    assert not unexplained

    # S2-S5 from the GPU's fp32 logits: bit-exact
    sel = oracle.selection_logits(L_gpu, b) if sel_only else L_gpu
    idx = oracle.select_topk(sel, w.k, G, M)
    gates = oracle.gate_weights(L_gpu, idx)
    tab = oracle.dispatch(idx, w.E, s.capacity,
                          slot_major=bool(flags & moe.MOE_FLAG_SLOT_MAJOR),
                          pad_to_capacity=bool(flags & moe.MOE_FLAG_PAD_TO_CAPACITY))
    R = moe.max_rows(s)
    assert np.array_equal(idx_gpu, idx)
    assert np.max(np.abs(lay.view("topk_w").cpu().numpy() - gates)) <= 1e-6
    assert np.array_equal(lay.routed_counts.cpu().numpy(), tab["routed_counts"])
    assert np.array_equal(lay.tokens_per_expert.cpu().numpy(), tab["tokens_per_expert"])
    assert np.array_equal(lay.view("offsets").cpu().numpy(), tab["expert_offsets"])
    assert np.array_equal(lay.view("dest_row").cpu().numpy(), tab["dest_row"])
    assert np.array_equal(lay.view("src_token").cpu().numpy(), tab["src_token"][:R])
    drops = lay.drops.cpu().numpy()
    assert drops[0] == tab["drops_total"]
    assert np.array_equal(drops[1:w.k + 1], tab["drops_per_slot"])
    assert drops[w.k + 1] == tab["fully_dropped_tokens"]
    assert int(lay.tokens_per_expert.sum()) == w.T * w.k - int(drops[0])  # conservation
    if flags & moe.MOE_FLAG_PAD_TO_CAPACITY:  # every empty slot holds a zero row
        empty = torch.from_numpy(np.nonzero(tab["src_token"][:R] < 0)[0]).cuda()
        assert torch.count_nonzero(lay.view("x_perm")[empty]).item() == 0
    log(f"  tables bit-exact: kept {tab['n_kept']} rows, dropped {tab['drops_total']}")

    # S9: the record of the layer's counts against the oracle's
    st = moe.expert_stats(w.T, w.k, lay.routed_counts.cpu().numpy(),
                          lay.tokens_per_expert.cpu().numpy())
    want = oracle.expert_stats(tab["routed_counts"], w.T, w.k, tab["tokens_per_expert"],
                               tab["drops_total"])
    for key in ("expert_p50", "expert_p95", "expert_max", "dropped_tokens"):
        assert st[key] == want[key], key
    assert abs(st["expert_max_to_mean"] - want["expert_max_to_mean"]) <= 1e-12

    # S6-S8: every output row
    out_gpu = to_host(lay.out)
    del lay
    torch.cuda.empty_cache()
    t0 = time.time()
    step = max(1, w.E // 8)

    def progress(e):
        if (e + 1) % step == 0:
            log(f"  oracle experts {e + 1}/{w.E} ({time.time() - t0:.0f} s)")

    Y = oracle.expert_ffn_streamed(x, tab["src_token"], tab["expert_offsets"], expert_weights(w),
                                   progress)
    want_out = oracle.combine(Y, tab["dest_row"], gates)
    err = rel_err(out_gpu, want_out)
    # a token whose every slot was dropped gets an exact zero row
    gone = np.all(tab["dest_row"] < 0, axis=1)
    assert not np.any(out_gpu[gone])
    row_err = np.max(np.abs(out_gpu - want_out), axis=1) / float(np.max(np.abs(want_out)))
    log(f"  all {w.T} rows: rel err {err:.3e} (worst row {int(np.argmax(row_err))}); "
        f"{int(gone.sum())} fully dropped tokens")
    assert err <= OUT_TOL
    return tab
