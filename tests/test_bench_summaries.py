# Host logic of bench.py's rocprofv3 summaries, on small synthetic CSV files in the layout
# rocprofv3 writes (agent info, kernel trace, counter collection).
import csv
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GATE_UP = "void moe::prefill_gemm_kernel<__bf16, true, moe::PrefillTileT<128, 2, 320>>(x)"
DOWN = "void moe::prefill_gemm_kernel<__bf16, false, moe::PrefillTileT<128, 2, 320>>(x)"
# the same template with bf16 operands and an fp32 output: router logits in dense mode
ROUTER = ("_ZN3moe19prefill_gemm_kernelIDF16bLb0ENS_12PrefillTileTILi128ELi3ELi64ELi128ELi2ELi4"
          "ELi0ELi0EEES2_fS2_EEvPKT_PKiS5_S5_lPT3_PKfPfiiS7_S7_iiiiiii")
# ... with one more tile type after the output type (two back-references), and a down GEMM
# whose output type is bf16 followed by back-references
ROUTER_PM = ("_ZN3moe19prefill_gemm_kernelIDF16bLb0ENS_12PrefillTileTILi128ELi3ELi64ELi128ELi2ELi4"
             "ELi0ELi0ELi0EEES2_fS2_S2_EEvPKT_PKiS5_S5_lPT3_PKfPfiiS7_S7_iiiiiii")
DOWN_PM = ("_ZN3moe19prefill_gemm_kernelIDF16bLb0ENS_12PrefillTileTILi128ELi2ELi256ELi256ELi2ELi4"
           "ELi1ELi3ELi1EEENS1_ILi128ELi2ELi128ELi256ELi2ELi4ELi1ELi3ELi2EEEDF16bS3_S2_EEvPKT_PKiS6_"
           "S6_lPT3_PKfPfiiS8_S8_iiiiiii")
COPY = "__amd_rocclr_copyBuffer"


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_counter_summary(bench, tmp_path):
    _write(tmp_path / "run_agent_info.csv",
           [{"Name": "AMD EPYC", "Cu_Count": "16", "Num_Xcc": "1", "Simd_Count": "0"},
            {"Name": "gfx950", "Cu_Count": "256", "Num_Xcc": "8", "Simd_Count": "1024"}])
    # dispatch 1: 1 ms at 1.7 GHz on 8 XCDs; 2: 0.5 ms at 2.4 GHz; 3: 2 ms at 1.8 GHz
    trace = [{"Dispatch_Id": "1", "Kernel_Name": GATE_UP, "Start_Timestamp": "0", "End_Timestamp": "1000000"},
             {"Dispatch_Id": "2", "Kernel_Name": DOWN, "Start_Timestamp": "0", "End_Timestamp": "500000"},
             {"Dispatch_Id": "3", "Kernel_Name": GATE_UP, "Start_Timestamp": "0", "End_Timestamp": "2000000"},
             {"Dispatch_Id": "4", "Kernel_Name": ROUTER, "Start_Timestamp": "0", "End_Timestamp": "100000"}]
    _write(tmp_path / "run_kernel_trace.csv", trace)
    # dispatch 1 also: MFMA units busy 60 % of the active clocks, 1.2e12 bf16 MFMA flops
    cc = [{"Dispatch_Id": "1", "Kernel_Name": GATE_UP, "Counter_Name": "GRBM_COUNT", "Counter_Value": str(1.7e6 * 8)},
          {"Dispatch_Id": "1", "Kernel_Name": GATE_UP, "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": str(1.7e6 * 8)},
          {"Dispatch_Id": "1", "Kernel_Name": GATE_UP, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES", "Counter_Value": str(0.6 * 1.7e6 * 1024)},
          {"Dispatch_Id": "1", "Kernel_Name": GATE_UP, "Counter_Name": "SQ_INSTS_VALU_MFMA_MOPS_BF16", "Counter_Value": str(1.2e12 / 512)},
          {"Dispatch_Id": "2", "Kernel_Name": DOWN, "Counter_Name": "GRBM_COUNT", "Counter_Value": str(2.4e6 / 2 * 8)},
          {"Dispatch_Id": "3", "Kernel_Name": GATE_UP, "Counter_Name": "GRBM_COUNT", "Counter_Value": str(1.8e6 * 2 * 8)},
          {"Dispatch_Id": "4", "Kernel_Name": ROUTER, "Counter_Name": "GRBM_COUNT", "Counter_Value": str(2.0e5 * 8)}]
    _write(tmp_path / "run_counter_collection.csv", cc)
    out = bench.summarize_counters(str(tmp_path))
    assert out["xcds"] == 8 and out["simds"] == 1024
    by = {k["kernel"]: k for k in out["kernels"]}
    gu = by["prefill_gemm_kernel (gate/up+SwiGLU)"]
    assert gu["dispatches"] == 2 and gu["median_us"] == 1500.0
    assert gu["clock_ghz"] == pytest.approx(1.75)
    # only dispatch 1 carries the MFMA counters
    assert gu["mfma_busy_pct"] == pytest.approx(60.0)
    assert gu["mfma_gflop_per_dispatch"] == pytest.approx(1200.0)
    assert gu["mfma_tflops"] == pytest.approx(1200.0, rel=1e-3)  # 1.2e12 flop in 1 ms
    dn = by["prefill_gemm_kernel (down)"]
    assert dn["clock_ghz"] == pytest.approx(2.4) and dn["median_us"] == 500.0
    rt = by["prefill_gemm_kernel (router logits, dense)"]
    assert rt["dispatches"] == 1 and rt["clock_ghz"] == pytest.approx(2.0)
    assert by["prefill_gemm_kernel (down)"]["dispatches"] == 1  # not merged with the router
    # the kernel with the most total time comes first
    assert out["kernels"][0]["kernel"] == "prefill_gemm_kernel (gate/up+SwiGLU)"


def test_traffic_summary(bench, tmp_path):
    kib_copy = bench.COPY_BYTES / 1024 * 0.5  # the counter reads half the copy's bytes
    for counter, sub, gate_kib in (("FETCH_SIZE", "fetch", [100.0, 300.0, 200.0]),
                                   ("WRITE_SIZE", "write", [50.0, 50.0, 50.0])):
        d = tmp_path / sub
        d.mkdir()
        rows = [{"Kernel_Name": COPY, "Counter_Name": counter, "Counter_Value": str(kib_copy)},
                {"Kernel_Name": COPY, "Counter_Name": counter, "Counter_Value": "4.0"},
                {"Kernel_Name": DOWN, "Counter_Name": counter, "Counter_Value": "9999.0"}]
        rows += [{"Kernel_Name": GATE_UP, "Counter_Name": counter, "Counter_Value": str(v)}
                 for v in gate_kib]
        _write(d / "run_counter_collection.csv", rows)
    out = bench.summarize_traffic(str(tmp_path / "fetch"), str(tmp_path / "write"), "wl")
    assert out["fetch_copy_factor"] == pytest.approx(0.5)
    # median 200 KiB, scaled by 1 / 0.5; the down GEMM's rows are not counted
    assert out["fetch_bytes_scaled"] == pytest.approx(200 * 1024 * 2)
    assert out["write_bytes_scaled"] == pytest.approx(50 * 1024 * 2)
    assert out["traffic_bytes"] == pytest.approx((200 + 50) * 1024 * 2)


def test_segment_drops(bench):
    # 5 tokens, k = 2; tokens 3 and 4 form the second segment, token 4 loses both slots
    dest = [[0, 1], [2, -1], [3, 4], [-1, 5], [-1, -1]]
    got = bench.segment_drops(dest, (("prefill", 0, 3), ("decode", 3, 5)))
    assert got == {"prefill": {"tokens": 3, "dropped": 1, "fully_dropped_tokens": 0},
                   "decode": {"tokens": 2, "dropped": 3, "fully_dropped_tokens": 1}}


def test_written_extent(bench):
    import torch

    buf = torch.full((200_000,), bench.SENTINEL, dtype=torch.uint8)
    assert bench.written_extent(buf) == 0
    buf[123_456] = 0
    assert bench.written_extent(buf) == 123_457
    buf[199_999] = 1  # past the last whole 64 KiB chunk
    assert bench.written_extent(buf) == 200_000
    small = torch.full((10,), bench.SENTINEL, dtype=torch.uint8)
    small[3] = 7
    assert bench.written_extent(small) == 4
    assert bench.written_extent(small[:0]) == 0


def test_rooflines(bench):
    import moe_inputs as mi

    # Mixtral-8x7B gate/up: 4 N d F flops over the event time, against 2500 TFLOP/s
    w = mi.WORKLOADS["mixtral_8x7b_prefill"]
    r = bench.gate_up_roofline(w, 8192, 8, 1.6204)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(4 * 8192 * 4096 * 14336 / 1.6204e-3 / 1e12, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / 2500.0, abs=1e-4)
    # DeepSeek-V3 decode: 8 rows per expert, far below the ridge: bytes against 8 TB/s
    w = mi.WORKLOADS["dsv3_decode"]
    r = bench.gate_up_roofline(w, 2048, 256, 2.0)
    want = 2 * (2 * 256 * 2048 * 7168 + 2048 * 7168 + 2048 * 2048) / 2e-3 / 1e9
    assert r["bound"] == "hbm" and r["achieved"] == pytest.approx(want, rel=1e-4)
    # layer: max(F_alg / P, B_alg / BW) over the step time
    w = mi.WORKLOADS["mixtral_8x7b_prefill"]
    F_alg = 2 * 4096 * 4096 * 8 + 6 * 4096 * 14336 * 8192
    assert bench.layer_roofline_frac(w, 8192, 8, 2.0) == pytest.approx(
        F_alg / 2.5e15 / 2e-3, abs=1e-4)


def test_trace_summary_splits_by_grid(bench, tmp_path):
    # the same GEMM kernel launched with two grids (two layers) is summarised per grid
    def row(i, name, grid, ns):
        return {"Dispatch_Id": str(i), "Kernel_Name": name, "Start_Timestamp": "0",
                "End_Timestamp": str(ns), "Grid_Size_X": str(grid * 512),
                "Workgroup_Size_X": "512"}
    _write(tmp_path / "x_kernel_trace.csv",
           [row(1, GATE_UP, 3136, 1_600_000), row(2, GATE_UP, 3136, 1_700_000),
            row(3, GATE_UP, 1536, 1_100_000), row(4, DOWN, 448, 800_000)])
    out = bench.summarize_trace(str(tmp_path))
    by = {(r["kernel"], r["blocks"]): r for r in out}
    a = by[("prefill_gemm_kernel (gate/up+SwiGLU)", 3136)]
    assert a["dispatches"] == 2 and a["mean_us"] == 1650.0 and a["min_us"] == 1600.0
    assert by[("prefill_gemm_kernel (gate/up+SwiGLU)", 1536)]["mean_us"] == 1100.0
    assert by[("prefill_gemm_kernel (down)", 448)]["total_ms"] == 0.8
    assert out[0]["blocks"] == 3136  # ordered by total time


def test_kernel_names(bench):
    assert bench._short_kernel(GATE_UP) == "prefill_gemm_kernel (gate/up+SwiGLU)"
    assert bench._short_kernel(DOWN) == "prefill_gemm_kernel (down)"
    assert bench._short_kernel(ROUTER) == "prefill_gemm_kernel (router logits, dense)"
    assert bench._short_kernel(ROUTER_PM) == "prefill_gemm_kernel (router logits, dense)"
    assert bench._short_kernel(DOWN_PM) == "prefill_gemm_kernel (down)"
    assert bench._short_kernel("_ZN3moe14combine_kernelIDF16bEEvPKT_") == "moe::combine_kernel"
    assert (bench._short_kernel("_ZN12_GLOBAL__N_116mfma_rate_kernelILi0EEEvijiPfPy")
            == "mfma_rate_kernel (calibration, 32x32x16)")
    assert (bench._short_kernel("void (anonymous namespace)::mfma_rate_kernel<1>(int)")
            == "mfma_rate_kernel (calibration, 16x16x32)")
    assert bench._short_kernel(COPY) == COPY
    assert bench._short_kernel("Cijk_Ailk_Bljk_BBS_BH_UserArgs") == "hipBLASLt GEMM (vendor reference)"


def test_power_summary(bench):
    """Polls that repeat one metric-table read count once; the first second of a phase and
    polls outside it are left out; unavailable fields ('N/A') are skipped."""
    samples = [(0.5, 240, 150.0, 45),      # before the phase
               (10.2, 900, 1300.0, 50),    # first second of the phase: skipped
               (11.2, 1376, 1972.5, 54), (11.25, 1376, 1972.5, 54), (11.3, 1376, 1972.5, 54),
               (12.2, 1390, 1960.0, 56),
               (13.2, 1380, "N/A", "N/A"),
               (15.0, 300, 200.0, 40)]     # after the phase
    out = bench.summarize_power(samples, [("layer", 10.0, 13.5)], 1400.0)
    rec = out["layer"]
    assert rec["refreshes"] == 3
    assert rec["socket_power_w"] == 1380
    assert rec["frac_of_cap"] == round(1380 / 1400.0, 3)
    assert rec["gfx_clock_mhz"] == round((1972.5 + 1960.0) / 2)
    assert rec["hotspot_c_max"] == 56
    assert out["power_cap_w"] == 1400.0
    empty = bench.summarize_power([], [("idle", 0.0, 2.0)], 1400.0)["idle"]
    assert empty["refreshes"] == 0 and empty["socket_power_w"] is None
