"""GPU check of the MFMA-rate calibration (libmoe_calib.so): the loop really computes the
bf16 products it counts, on the operands it claims, so its flop count is honest.

Each wave accumulates, for 4 chains, iters times the product C = A B^T of its register
operands: 32x32 with k = 16 (lane l holds row l % 32 of A and of B at k = 8 (l / 32) ..
8 (l / 32) + 7), or 16x16 with k = 32 (row l % 16, k = 8 (l / 16) .. 8 (l / 16) + 7).  The
sum of all elements of C is sum_k (sum_m A[m, k]) (sum_n B[n, k]), which the host computes
from the same hash; a wave's sink value is iters times the sum over its 4 chains."""
import numpy as np
import pytest

import routing_expert_ffn_router_amd as moe

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

WAVES, CHAINS = 8, 4


def hash32(x):
    x = x.astype(np.uint64) & 0xFFFFFFFF
    x ^= x >> 16
    x = (x * 0x85EBCA6B) & 0xFFFFFFFF
    x ^= x >> 13
    x = (x * 0xC2B2AE35) & 0xFFFFFFFF
    x ^= x >> 16
    return x


def bf16_value(half):
    """The bf16 value of a 16-bit pattern the kernel builds: sign bit 15, mantissa bits 0-6
    and the exponent 125 + (bits 7-8), as float64 (exact)."""
    sign = np.where(half & 0x8000, -1.0, 1.0)
    exp = 125 + ((half >> 7) & 3)
    mant = half & 0x7F
    return sign * (1.0 + mant / 128.0) * np.exp2(exp.astype(np.float64) - 127)


def expected_sink(blocks, iters, seed, shape=0):
    """Each wave's exact sink value, and a bound on its fp32 rounding error."""
    want = np.zeros(blocks * WAVES)
    bound = np.zeros(blocks * WAVES)
    lane = np.arange(64, dtype=np.uint64)
    kbase = (8 * (lane // (32 if shape == 0 else 16))).astype(np.int64)
    for blk in range(blocks):
        for wave in range(WAVES):
            total = absum = 0.0
            for j in range(CHAINS):
                col = {n: np.zeros(32) for n in ("a", "b", "|a|", "|b|")}
                for q in range(4):
                    ctr = ((blk * WAVES + wave) * 64 + lane) * (2 * CHAINS * 4) + (j * 4 + q) * 2
                    for name, h in (("a", hash32(ctr ^ seed)), ("b", hash32((ctr + 1) ^ seed))):
                        for e, half in ((2 * q, h & 0xFFFF), (2 * q + 1, (h >> 16) & 0xFFFF)):
                            v = bf16_value(half)
                            np.add.at(col[name], kbase + e, v)
                            np.add.at(col["|" + name + "|"], kbase + e, np.abs(v))
                total += float(np.dot(col["a"], col["b"]))
                absum += float(np.dot(col["|a|"], col["|b|"]))
            want[blk * WAVES + wave] = iters * total
            # 16- or 32-term MFMA sums, iters accumulations, 16 + 64 terms per wave: < 64 u
            bound[blk * WAVES + wave] = 64 * 2.0 ** -24 * iters * absum
    return want, bound


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load_calib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("shape", [0, 1])
def test_calib_mfma_computes_the_counted_products(shape):
    blocks, iters, seed = 4, 3, 12345
    sink = torch.full((blocks * WAVES,), float("nan"), device="cuda")
    cyc = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    moe.calib_mfma(blocks, iters, seed, True, sink, cyc, shape=shape)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().astype(np.float64)
    want, bound = expected_sink(blocks, iters, seed, shape)
    assert np.all(np.abs(got - want) <= bound), (got[:4], want[:4], bound[:4])
    assert np.all(np.abs(want) > bound)  # the check has teeth
    c = cyc.view(blocks, 2).cpu().numpy()
    assert np.all(c > 0)
    # repeated with the same seed: the same values bit for bit
    sink2 = torch.empty_like(sink)
    moe.calib_mfma(blocks, iters, seed, True, sink2, cyc, shape=shape)
    torch.cuda.synchronize()
    assert torch.equal(sink, sink2)


def test_calib_mfma_zero_operands_and_clock():
    blocks = 2
    sink = torch.full((blocks * WAVES,), float("nan"), device="cuda")
    cyc = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    moe.calib_mfma(blocks, 2000, 7, False, sink, cyc)
    torch.cuda.synchronize()
    assert torch.count_nonzero(sink).item() == 0
    khz = moe.calib_wall_clock_khz()
    assert khz > 0
    c = cyc.view(blocks, 2).sum(dim=0).tolist()
    ghz = c[0] / c[1] * khz * 1e3 / 1e9
    assert 0.3 < ghz < 3.5, ghz  # a shader clock, not the constant-rate counter
