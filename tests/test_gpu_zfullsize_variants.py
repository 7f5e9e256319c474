"""GPU parity of the routing and dispatch variants at full layer sizes, in the launch
configuration bench.py times them: the dispatch tables bit for bit over all T*k assignments
(the oracle routing from the GPU's fp32 logits) and the outputs of sampled tokens, which the
oracle computes one token at a time with the expert weights regenerated slice by slice."""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
import routing_expert_ffn_router_amd as moe
from _util import OUT_TOL, device_inputs, log, logits_tol, rel_err, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

PAD, SLOT, SEL = (moe.MOE_FLAG_PAD_TO_CAPACITY, moe.MOE_FLAG_SLOT_MAJOR,
                  moe.MOE_FLAG_BIAS_SELECTION_ONLY)
CASES = [  # workload, flags, n_groups, topk_groups
    ("mixtral_8x7b_prefill", PAD, 0, 0),
    ("dsv3_mixed", SLOT, 0, 0),
    ("dsv3_decode", 0, 8, 4),
    ("mixtral_8x22b_zipf", SEL, 0, 0),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,flags,G,M", CASES)
def test_fullsize_variant(name, flags, G, M):
    w = mi.WORKLOADS[name]
    log(f"full-size {name} flags={flags} groups={G}/{M}")
    C = moe.capacity(w.T, w.k, w.E, w.capacity_factor)
    s = moe.shape(w.T, w.d, w.E, w.k, w.F, C, moe.MOE_BF16, flags=flags, n_groups=G,
                  topk_groups=M)
    dev = device_inputs(w)
    lay = moe.MoELayer(s)
    lay(dev["x"], dev["w_router"], dev["b_router"], dev["w_gate"], dev["w_up"], dev["w_down"])
    torch.cuda.synchronize()
    del dev
    torch.cuda.empty_cache()
    assert lay.status.item() == 0
    sel_only = bool(flags & SEL)
    b = mi.router_bias(w)
    x = mi.host_tensor_f32(w, "x")
    L_ref = oracle.router_logits(x, mi.host_tensor_f32(w, "w_router"), None if sel_only else b)
    L_gpu = lay.view("logits").cpu().numpy()
    assert float(np.max(np.abs(L_gpu - L_ref))) <= logits_tol(L_ref)
    sel = oracle.selection_logits(L_gpu, b) if sel_only else L_gpu
    idx = oracle.select_topk(sel, w.k, G, M or None)
    gates = oracle.gate_weights(L_gpu, idx)
    tab = oracle.dispatch(idx, w.E, C, slot_major=bool(flags & SLOT),
                          pad_to_capacity=bool(flags & PAD))
    assert np.array_equal(lay.view("topk_idx").cpu().numpy(), idx)
    assert np.array_equal(lay.view("dest_row").cpu().numpy(), tab["dest_row"])
    assert np.array_equal(lay.view("offsets").cpu().numpy(), tab["expert_offsets"])
    assert np.array_equal(lay.view("src_token").cpu().numpy(),
                          tab["src_token"][:moe.max_rows(s)])
    drops = lay.drops.cpu().numpy()
    assert drops[0] == tab["drops_total"] and drops[w.k + 1] == tab["fully_dropped_tokens"]
    assert np.max(np.abs(lay.view("topk_w").cpu().numpy() - gates)) <= 1e-6
    if flags & PAD:  # empty slots hold zero rows
        empty = np.nonzero(tab["src_token"] < 0)[0]
        pick = torch.from_numpy(empty[np.linspace(0, len(empty) - 1, 16).astype(np.int64)]).cuda()
        assert torch.count_nonzero(lay.view("x_perm")[pick]).item() == 0
    cand = [0, 1, w.T // 3, w.T // 2, w.T - 1] + [seg[2] - 1 for seg in w.segments]
    toks = sorted(set(cand))[: (6 if w.E > 8 else 8)]
    kept = tab["dest_row"][toks] >= 0

    def weights(e):
        return (mi.host_tensor_f32(w, "w_gate", e, 1)[0], mi.host_tensor_f32(w, "w_up", e, 1)[0],
                mi.host_tensor_f32(w, "w_down", e, 1)[0])

    want = oracle.token_outputs(x[toks], idx[toks], kept, gates[toks], weights)
    got = to_host(lay.out[torch.tensor(toks, device="cuda")])
    err = rel_err(got, want)
    log(f"  drops {int(drops[0])}, sampled tokens {toks}: rel err {err:.3e}")
    assert err <= OUT_TOL
    del lay
    torch.cuda.empty_cache()
