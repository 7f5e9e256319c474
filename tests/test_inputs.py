"""The seeded input generator: Philox known answers, host build == numpy, moments."""
import json
import math
import os

import numpy as np
import pytest

import moe_inputs as mi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    kat = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    for v in kat["vectors"]:
        c = [np.array([int(h, 16)], dtype=np.uint64) for h in v["ctr"]]
        k0, k1 = (int(h, 16) for h in v["key"])
        out = mi.philox4x32_10_np(*c, k0, k1)
        assert [f"{int(o[0]):08x}" for o in out] == v["out"]


@pytest.mark.parametrize("start", [0, 12345, (1 << 32) - 7, (1 << 40) + 3])
@pytest.mark.parametrize("bf16", [False, True])
def test_host_fill_matches_numpy(start, bf16):
    n = 5000
    std = 0.0125
    ref = mi.values_np(mi.SEED, mi.TENSOR_IDS["w_gate"], start, n, mi.normal_scale(std))
    got = mi.host_values(mi.TENSOR_IDS["w_gate"], start, n, std, bf16)
    if bf16:
        assert np.array_equal(got, mi.bf16_rne_np(ref))
    else:
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_moments_and_range():
    std = 1.0 / math.sqrt(4096)
    v = mi.host_values_f32(mi.TENSOR_IDS["w_up"], 0, 2_000_000, std, False)
    assert abs(v.mean()) < 5 * std / math.sqrt(v.size)
    assert abs(v.std() / std - 1.0) < 3e-3
    # Irwin-Hall with n = 8 is bounded by sqrt(3 * 8) standard deviations.
    assert np.abs(v).max() <= math.sqrt(24.0) * std * (1 + 1e-6)


def test_streams_differ_and_are_deterministic():
    a = mi.host_values(1, 0, 1000, 1.0, False)
    b = mi.host_values(2, 0, 1000, 1.0, False)
    c = mi.host_values(1, 0, 1000, 1.0, False)
    assert not np.array_equal(a, b)
    assert np.array_equal(a, c)


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, 1.0 + 2.0**-8 + 2.0**-20, -2.5],
                 dtype=np.float32)
    got = mi.bf16_rne_np(f)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6)
    want = np.array([0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020], dtype=np.uint16)
    assert np.array_equal(got, want)
    assert np.array_equal(mi.bf16_bits_to_f32(want)[[0, 4]], np.array([1.0, -2.5], np.float32))


def test_zipf_bias():
    b = mi.zipf_bias(8, 1.1)
    assert b[0] == 0.0
    assert np.allclose(b.astype(np.float64), -1.1 * np.log(np.arange(1, 9)), rtol=1e-7)
    assert np.all(np.diff(b) < 0)


def test_workload_shapes():
    w = mi.WORKLOADS["dsv3_decode"]
    assert mi.tensor_shape(w, "w_gate") == (256, 2048, 7168)
    assert mi.tensor_shape(w, "w_down") == (256, 7168, 2048)
    tiny = mi.WORKLOADS["tiny_f32"]
    x = mi.host_tensor_f32(tiny, "x")
    assert x.shape == (64, 128) and x.dtype == np.float32
    wg = mi.host_tensor_f32(tiny, "w_gate", 3, 2)
    full = mi.host_tensor_f32(tiny, "w_gate")
    assert np.array_equal(wg, full[3:5])
