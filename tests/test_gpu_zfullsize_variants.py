"""GPU parity of the routing and dispatch variants at full layer sizes, in the launch
configuration bench.py times them: the dispatch tables bit for bit over all T*k assignments
(the oracle routing from the GPU's fp32 logits) and every output row, which the oracle
computes with each expert's weights regenerated one expert at a time."""
import pytest

import moe_inputs as mi
import routing_expert_ffn_router_amd as moe
from _fullsize import check_layer_every_token
from _util import log

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
    log(f"full-size {name} flags={flags} groups={G}/{M}: every token")
    C = moe.capacity(w.T, w.k, w.E, w.capacity_factor)
    s = moe.shape(w.T, w.d, w.E, w.k, w.F, C, moe.MOE_BF16, flags=flags, n_groups=G,
                  topk_groups=M)
    check_layer_every_token(w, s, torch)
