"""GPU parity of the routing and dispatch variants at full layer sizes, in the launch
configuration bench.py times them: the dispatch tables bit for bit over all T*k assignments
(the oracle routing from the GPU's fp32 logits) and every output row, which the oracle
computes with each expert's weights regenerated one expert at a time.  Also the layers
bench.py times as HIP graph replays: every replay equals the eager layer bit for bit."""
import pytest

import moe_inputs as mi
import routing_expert_ffn_router_amd as moe
from _fullsize import check_layer_every_token
from _util import device_inputs, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

PAD, SLOT, SEL = (moe.MOE_FLAG_PAD_TO_CAPACITY, moe.MOE_FLAG_SLOT_MAJOR,
                  moe.MOE_FLAG_BIAS_SELECTION_ONLY)
CASES = [  # workload, flags, n_groups, topk_groups: every variant bench.py times
    ("mixtral_8x7b_prefill", PAD, 0, 0),
    ("mixtral_8x22b_zipf", PAD, 0, 0),
    ("mixtral_8x22b_zipf", SLOT, 0, 0),
    ("mixtral_8x22b_zipf", SEL, 0, 0),
    ("dsv3_decode", 0, 8, 4),
    ("dsv3_mixed", PAD, 0, 0),
    ("dsv3_mixed", SLOT, 0, 0),
    ("dsv3_mixed", 0, 8, 4),
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
    log(f"full-size {name} flags={flags} groups={G}/{M}: every token")
    C = moe.capacity(w.T, w.k, w.E, w.capacity_factor)
    s = moe.shape(w.T, w.d, w.E, w.k, w.F, C, moe.MOE_BF16, flags=flags, n_groups=G,
                  topk_groups=M)
    check_layer_every_token(w, s, torch)


@pytest.mark.parametrize("name", ["mixtral_8x7b_prefill", "dsv3_decode", "dsv3_mixed"])
def test_fullsize_graph_replay_matches_eager(name):
    # moe_layer captured once and replayed three times, with eager layers of the program
    # between the replays; each replay's output, counts and tables equal the eager layer's
    w = mi.WORKLOADS[name]
    log(f"full-size {name}: graph replays against the eager layer")
    s = moe.shape(w.T, w.d, w.E, w.k, w.F, moe.capacity(w.T, w.k, w.E, w.capacity_factor),
                  moe.MOE_BF16)
    dev = device_inputs(w)
    args = (dev["x"], dev["w_router"], dev["b_router"], dev["w_gate"], dev["w_up"],
            dev["w_down"])
    eager = moe.MoELayer(s)
    eager(*args)
    lay = moe.MoELayer(s)
    lay(*args)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lay(*args)
    for rep in range(3):
        lay.out.fill_(0)
        lay.routed_counts.fill_(-1)
        eager(*args)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lay.out, eager.out), f"replay {rep}"
        assert torch.equal(lay.routed_counts, eager.routed_counts)
        assert torch.equal(lay.tokens_per_expert, eager.tokens_per_expert)
        assert torch.equal(lay.drops, eager.drops)
        assert torch.equal(lay.view("dest_row"), eager.view("dest_row"))
    log(f"  3 replays bit-exact ({int(eager.tokens_per_expert.sum())} kept rows)")
    del g, lay, eager, dev
    torch.cuda.empty_cache()
