"""GPU parity of the Mixtral-8x22B Zipf layer at the capacity factors bench.py sweeps
([EP-checks] "Capacity factor changes quality, memory and tail latency"), every token.

Each capacity changes how many rows the hot experts keep, and with it the GEMM plan: at
CF 1.0 (C = 512) both tile heights need two row tiles and the 256-row tile pads fewer rows;
at 1.5 and 2.0 the hottest experts hold two or three full 320-row tiles and a short tail that
runs double width; without a limit expert 0 keeps 1542 rows (four full tiles and a 262-row
one).  The down GEMM's tail split then sees a different tile count each time.  The default
factor (1.25) is covered by the full-size default-path test.
"""
import pytest

import moe_inputs as mi
import routing_expert_ffn_router_amd as moe
from _fullsize import check_layer_every_token
from _util import log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FACTORS = [1.0, 1.5, 2.0, None]  # None: no capacity limit (C = T)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cf", FACTORS)
def test_fullsize_capacity_factor(cf):
    w = mi.WORKLOADS["mixtral_8x22b_zipf"]
    C = moe.capacity(w.T, w.k, w.E, cf)  # 0 for no limit
    log(f"full-size {w.name} capacity factor {cf} (C={C}): every token")
    s = moe.shape(w.T, w.d, w.E, w.k, w.F, C, moe.MOE_BF16)
    tab = check_layer_every_token(w, s, torch)
    kept = tab["tokens_per_expert"]
    if cf is None:
        assert int(tab["drops_total"]) == 0
        assert int(kept.max()) == int(tab["routed_counts"].max())
    else:
        assert int(kept.max()) <= C
