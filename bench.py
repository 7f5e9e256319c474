#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X: tokens/s of route + dispatch + expert GEMMs + combine.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one moe_layer call (router logits, top-k gating, dispatch with capacity
truncation, grouped SwiGLU expert FFN, combine) over the workload's T tokens, with every
input already resident in HBM.  W untimed steps, then exactly K timed steps between
device synchronisations.  Prints one JSON line.

A second pass runs the same layer as its five ABI calls with HIP events between them:
it yields the per-stage timing record (router / pack / expert compute / unpack, as in
airouter.kz, "Expert parallelism in MoE needs measurements before launch", section
"All-to-all must be profiled separately from compute") and the duration of the dominant
kernel, from which the roofline fraction is computed.  The CPU oracle, timed on a bounded
sample of the same workload, is reported as a baseline.  The default run also times the other
workloads, sweeps the capacity factor of the skewed Mixtral-8x22B layer, and reports reference
points measured on the same GPU outside the timed region: hipBLASLt on the dense equivalents
of the two GEMMs, a device copy, the bf16 MFMA rate and clock the chip sustains
(--mfma-ceiling), and the socket power and graphics clock while the layer and that MFMA loop
run (--power).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s (route+dispatch+expert GEMM+combine), % MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3  # MI355X fp32 matrix/vector
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
DEFAULT_WORKLOAD = "mixtral_8x7b_prefill"
CPU_SAMPLE_TOKENS = {"mixtral_8x7b_prefill": 4096, "mixtral_8x22b_zipf": 512,
                     "dsv3_decode": 64, "dsv3_mixed": 256, "tiny_f32": 64}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=None,
                   help="tokens in the oracle's timed sample (default per workload)")
    p.add_argument("--pad", action="store_true",
                   help="pad-to-capacity dispatch: every expert owns C row slots")
    p.add_argument("--slot-major", action="store_true",
                   help="slot-major drop priority (first choices before second choices)")
    p.add_argument("--bias-selection-only", action="store_true",
                   help="the router bias shifts the selection only, not the gates")
    p.add_argument("--groups", default=None, metavar="G:M",
                   help="group-limited top-k: G expert groups, M kept per token")
    p.add_argument("--capacity-factor", type=float, default=None,
                   help="override the workload's capacity factor (<= 0: no limit)")
    p.add_argument("--cf-sweep", default=None, metavar="CF,CF,...",
                   help="also time the layer at each capacity factor ('none': no limit)")
    p.add_argument("--other-steps", type=int, default=10,
                   help="timed steps of each other workload in the default run")
    p.add_argument("--no-other-workloads", action="store_true",
                   help="time the headline workload only")
    p.add_argument("--ep", type=int, default=8,
                   help="ranks of the expert placement in the routing record (contiguous)")
    p.add_argument("--ranks-per-node", type=int, default=8)
    p.add_argument("--graph", action="store_true",
                   help="time replays of a HIP graph that captured one moe_layer call")
    p.add_argument("--mfma-ceiling", nargs="?", const="both", default=None,
                   choices=["both", "random", "zero"],
                   help="only measure the sustained bf16 MFMA rate and clock (libmoe_calib.so) "
                        "on random and/or all-zero operands")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a device copy of known size (for rocprofv3 --pmc scaling)")
    p.add_argument("--summarize-counters", metavar="PMC_DIR",
                   help="per kernel of a rocprofv3 --pmc ... --kernel-trace run: shader clock "
                        "(GRBM_COUNT), MFMA busy share (SQ_VALU_MFMA_BUSY_CYCLES over "
                        "GRBM_GUI_ACTIVE) and bf16 MFMA flops (SQ_INSTS_VALU_MFMA_MOPS_BF16), "
                        "for whichever of these counters the run holds")
    p.add_argument("--summarize-trace", metavar="TRACE_DIR",
                   help="per kernel and grid of a rocprofv3 --kernel-trace run: dispatches and "
                        "mean / median / min / max duration")
    p.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                        "script into profiles/traffic_<workload>.json and exit")
    p.add_argument("--power", action="store_true",
                   help="only record socket power and graphics clock (driver metrics) while "
                        "the GPU idles, loops the headline layer, the MFMA calibration loop "
                        "and the decode layer, then exit")
    return p.parse_args()


COPY_BYTES = 512 << 20  # bytes read (and written) by the calibration copy
KERNEL_SOURCES = ["routing_expert_ffn_router_amd/csrc/expert_ffn.hip",
                  "routing_expert_ffn_router_amd/csrc/common.h"]


def kernel_source_sha() -> str:
    """Hash of the GEMM kernel's code with comments and whitespace removed, so the traffic
    counters stay attached to the kernel across comment edits."""
    import hashlib
    import re

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        src = open(os.path.join(ROOT, f)).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def _pmc_rows(d):
    import csv
    import glob

    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    return rows


# The two counter runs a traffic summary is made from (R: the repository root, OUT: the folder,
# relative to R, that receives the profiler's output), then the summary itself.
TRAFFIC_COMMANDS = [
    "cd /tmp && export TMPDIR=/tmp && timeout -s KILL 150 rocprofv3 --pmc {c} --kernel-trace "
    "--output-format csv -d $R/$OUT/prof/{t}_{w} -o run -- python3 $R/bench.py "
    "--no-cpu-baseline --steps 5 --warmup 2 --no-other-workloads --workload {w} "
    "--copy-calibration",
    "cd $R && python3 bench.py --workload {w} --summarize-traffic $OUT/prof/fetch_{w} "
    "$OUT/prof/write_{w}",
]


def summarize_traffic(fetch_dir, write_dir, workload):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the dominant kernel, scaled by what the
    same counters read for the calibration copy of COPY_BYTES."""
    import statistics as st

    out = {"workload": workload, "kernel_source_sha": kernel_source_sha(),
           "copy_bytes": COPY_BYTES,
           "commands": [TRAFFIC_COMMANDS[0].format(c=c, t=t, w=workload)
                        for c, t in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write"))] +
                       [TRAFFIC_COMMANDS[1].format(w=workload)]}
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = [r for r in _pmc_rows(d) if r["Counter_Name"] == counter]
        copy = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        # the gate/up GEMM is the grouped GEMM instantiated with SwiGLU on (the down GEMM's
        # name carries the false / Lb0E template argument)
        gate_up = [r for r in rows if "prefill_gemm_kernel" in r["Kernel_Name"] and
                   "Lb0E" not in r["Kernel_Name"] and "false" not in r["Kernel_Name"]]
        if not copy or not gate_up:
            raise SystemExit(f"{counter}: no copy or gate/up kernel rows in {d}")
        kib_copy = max(copy)  # the calibration copies are the largest copies of the run
        factor = kib_copy * 1024.0 / COPY_BYTES
        kib = st.median(float(r["Counter_Value"]) for r in gate_up)
        out[f"{key}_kib_per_dispatch"] = kib
        out[f"{key}_copy_kib"] = kib_copy
        out[f"{key}_copy_factor"] = round(factor, 4)
        out[f"{key}_bytes_scaled"] = kib * 1024.0 / factor
        out["kernel"] = gate_up[0]["Kernel_Name"][:120]
    out["traffic_bytes"] = out["fetch_bytes_scaled"] + out["write_bytes_scaled"]
    return out


def summarize_counters(d):
    """Per kernel, medians over its dispatches of the derived figures the run's counters
    allow.  GRBM_COUNT and GRBM_GUI_ACTIVE count GPU clocks on every XCD (rocprofv3 reports
    the sum), SQ_VALU_MFMA_BUSY_CYCLES counts busy cycles of every SIMD's MFMA unit, and
    SQ_INSTS_VALU_MFMA_MOPS_BF16 counts bf16 MFMA work in units of 512 flops:
        clock_ghz     = GRBM_COUNT / XCDs / duration
        mfma_busy_pct = 100 * SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs * SIMDs)
        mfma_tflops   = 512 * SQ_INSTS_VALU_MFMA_MOPS_BF16 / duration
    and, where the run holds them, the LDS bank-conflict share of the LDS cycles
    (SQ_LDS_BANK_CONFLICT over SQ_LDS_IDX_ACTIVE) and the L2 hit rate (TCC_HIT over
    TCC_HIT + TCC_MISS)."""
    import csv
    import glob
    import statistics as st

    def rows(pattern):
        out = []
        for f in glob.glob(os.path.join(d, "**", pattern), recursive=True):
            out += list(csv.DictReader(open(f)))
        return out

    agents = [r for r in rows("*agent_info.csv") if r.get("Name", "").startswith("gfx")]
    if not agents:
        raise SystemExit(f"no GPU agent in {d}")
    n_xcc, n_simd = int(agents[0]["Num_Xcc"]), int(agents[0]["Simd_Count"])
    span = {r["Dispatch_Id"]: int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            for r in rows("*kernel_trace.csv")}
    disp = {}
    for r in rows("*counter_collection.csv"):
        did = r["Dispatch_Id"]
        if did not in span or span[did] <= 0:
            continue
        e = disp.setdefault(did, {"name": r["Kernel_Name"], "ns": span[did]})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])

    per = {}
    for e in disp.values():
        ns = e["ns"]
        f = {"ns": ns}
        if "GRBM_COUNT" in e:
            f["clock_ghz"] = e["GRBM_COUNT"] / n_xcc / ns
        if "SQ_VALU_MFMA_BUSY_CYCLES" in e and e.get("GRBM_GUI_ACTIVE"):
            f["mfma_busy_pct"] = (100.0 * e["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                  (e["GRBM_GUI_ACTIVE"] / n_xcc * n_simd))
        if "SQ_LDS_BANK_CONFLICT" in e and e.get("SQ_LDS_IDX_ACTIVE"):
            f["lds_bank_conflict_pct"] = (100.0 * e["SQ_LDS_BANK_CONFLICT"] /
                                          e["SQ_LDS_IDX_ACTIVE"])
        hit, miss = e.get("TCC_HIT_sum", e.get("TCC_HIT")), e.get("TCC_MISS_sum",
                                                                   e.get("TCC_MISS"))
        if hit is not None and miss is not None and hit + miss > 0:
            f["l2_hit_pct"] = 100.0 * hit / (hit + miss)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in e:
            f["mfma_tflops"] = 512.0 * e["SQ_INSTS_VALU_MFMA_MOPS_BF16"] / ns / 1e3
            f["mfma_gflop_per_dispatch"] = 512.0 * e["SQ_INSTS_VALU_MFMA_MOPS_BF16"] / 1e9
        per.setdefault(_short_kernel(e["name"]), []).append(f)
    out = []
    for name, v in sorted(per.items(), key=lambda kv: -sum(f["ns"] for f in kv[1])):
        k = {"kernel": name, "dispatches": len(v),
             "median_us": round(st.median(f["ns"] for f in v) / 1e3, 1)}
        for key, nd in (("clock_ghz", 3), ("mfma_busy_pct", 1), ("mfma_tflops", 1),
                        ("mfma_gflop_per_dispatch", 2), ("lds_bank_conflict_pct", 2),
                        ("l2_hit_pct", 1)):
            vals = [f[key] for f in v if key in f]
            if vals:
                k[key] = round(st.median(vals), nd)
        out.append(k)
    return {"xcds": n_xcc, "simds": n_simd, "kernels": out}


def _short_kernel(name):
    """Readable name of a kernel of this library (the grouped GEMM by its role)."""
    import re

    if "prefill_gemm_kernel" in name:
        # bf16 operands with an fp32 output: the router logits in dense mode (mangled: the
        # output type f, possibly followed by back-references to the tile types, closes the
        # template arguments; demangled: ", float" among them)
        if ("IDF16b" in name and re.search(r"f(?:S\d*_)*EEvPKT_", name)) or (
                "__bf16" in name and re.search(r", float[,>]", name)):
            return "prefill_gemm_kernel (router logits, dense)"
        return "prefill_gemm_kernel (" + (
            "down" if "Lb0E" in name or "false" in name else "gate/up+SwiGLU") + ")"
    m = re.match(r"_ZN(\d+)moe(\d+)", name)  # mangled moe::<name><template args>
    if m:
        start = m.end()
        return "moe::" + name[start:start + int(m.group(2))]
    if name.startswith("Cijk_"):  # hipBLASLt's GEMM in the vendor reference
        return "hipBLASLt GEMM (vendor reference)"
    if "mfma_rate_kernel" in name:  # the calibration loop (libmoe_calib.so)
        one = "ILi1E" in name or "<1>" in name
        return "mfma_rate_kernel (calibration, " + ("16x16x32)" if one else "32x32x16)")
    return name.split("(")[0].split("<")[0].replace("void ", "")


def summarize_trace(d):
    """Per (kernel, grid) of a rocprofv3 --kernel-trace run: dispatches and their mean,
    median, min and max duration.  The grid tells apart layers that launch the same kernel
    (the Mixtral-8x7B and -8x22B GEMMs share one template instance)."""
    import csv
    import glob
    import statistics as st

    rows = []
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    if not rows:
        raise SystemExit(f"no kernel trace in {d}")
    per = {}
    for r in rows:
        ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        grid = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0)
        wg = int(r.get("Workgroup_Size_X") or r.get("Workgroup_Size") or 1)
        key = (_short_kernel(r["Kernel_Name"]), grid // max(wg, 1), wg)
        per.setdefault(key, []).append(ns)
    out = []
    for (name, blocks, wg), v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        out.append({"kernel": name, "blocks": blocks, "block_threads": wg,
                    "dispatches": len(v), "mean_us": round(st.mean(v) / 1e3, 1),
                    "median_us": round(st.median(v) / 1e3, 1),
                    "min_us": round(min(v) / 1e3, 1), "max_us": round(max(v) / 1e3, 1),
                    "total_ms": round(sum(v) / 1e6, 3)})
    return out


def traffic_for(workload):
    """Scaled HBM bytes per gate/up launch from the committed summary, or None when the
    kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t["traffic_bytes"]


def build_if_missing():
    import __graft_entry__

    __graft_entry__._ensure_built()


def segment_drops(dest_row, segments) -> dict:
    """Drops per named token range ([EP-checks] "Top-2 does not insure against hot experts":
    look at who loses when experts overflow).  dest_row is the [T, k] table of the layer (-1
    for a dropped assignment); segments are (name, first token, end token)."""
    import numpy as np

    out = {}
    for name, t0, t1 in segments:
        rows = np.asarray(dest_row[t0:t1])
        out[name] = {"tokens": int(t1 - t0), "dropped": int((rows < 0).sum()),
                     "fully_dropped_tokens": int(np.all(rows < 0, axis=1).sum())}
    return out


def percentile(v, q):
    s = sorted(v)
    return s[min(len(s) - 1, max(0, math.ceil(q * len(s)) - 1))]


def cpu_baseline(w, ntok: int) -> dict:
    """The oracle, as it stands, on the first `ntok` tokens of the workload (capacity
    recomputed for ntok tokens with the same factor), full router and expert weights.  Its
    steps run one by one (the same calls its moe_layer makes) so each stage is timed."""
    import numpy as np
    import threadpoolctl

    import moe_inputs as mi
    import oracle

    x = mi.host_tensor_f32(w, "x", 0, ntok)
    wr = mi.host_tensor_f32(w, "w_router")
    b = mi.router_bias(w)
    wg, wu, wd = (mi.host_tensor_f32(w, n) for n in ("w_gate", "w_up", "w_down"))
    C = oracle.capacity(ntok, w.k, w.E, w.capacity_factor)
    stages = {}
    t0 = time.perf_counter()

    def lap(name):
        nonlocal t0
        t = time.perf_counter()
        stages[name] = round(t - t0, 4)
        t0 = t

    L = oracle.router_logits(x, wr, b)
    lap("router_s")
    idx = oracle.select_topk(L, w.k)
    gates = oracle.gate_weights(L, idx)
    lap("topk_s")
    tab = oracle.dispatch(idx, w.E, C)
    xp = oracle.permute(x, tab["src_token"], tab["n_kept"])
    lap("dispatch_s")
    Y = oracle.expert_ffn(xp, tab["expert_offsets"], wg, wu, wd)
    lap("expert_ffn_s")
    out = oracle.combine(Y, tab["dest_row"], gates)
    lap("combine_s")
    dt = sum(stages.values())
    assert np.all(np.isfinite(out))
    threads = 0
    for info in threadpoolctl.threadpool_info():
        threads = max(threads, int(info.get("num_threads", 0)))
    return {"value": ntok / dt, "unit": "tokens/s", "cores": threads or os.cpu_count(),
            "kind": "oracle", "seconds": round(dt, 3), "stage_seconds": stages,
            "sample": f"first {ntok} of {w.T} tokens of {w.name}, all {w.E} experts, "
                      f"capacity {C} (same factor), float64 numpy oracle",
            "cpu_model": _cpu_model()}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def gate_up_roofline(w, N, E_active, t_ms) -> dict:
    """Roofline of the gate/up grouped GEMM (the dominant kernel): algorithmic flops 4 N d F
    against the dtype's MFMA peak, or, below the ridge, algorithmic bytes
    b (2 E_active F d + N d + N F) against HBM, over its event-timed duration."""
    t = t_ms * 1e-3
    flops = 4.0 * N * w.d * w.F
    nbytes = w.elt_bytes * (2.0 * E_active * w.F * w.d + N * w.d + N * w.F)
    peak = (PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS) * 1e12
    if nbytes == 0 or t <= 0:
        return {"bound": "mfma", "achieved": 0.0, "peak": peak / 1e12, "unit": "TFLOP/s",
                "frac": 0.0}
    if flops / nbytes >= peak / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": round(flops / t / 1e12, 2), "peak": peak / 1e12,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(nbytes / t / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    return roof


def layer_roofline_frac(w, N, E_active, ms) -> float:
    """t_roof / t_step with t_roof = max(F_alg / P, B_alg / BW) over the whole layer:
    F_alg = 2 T d E + 6 d F N, B_alg = b (2 T d + E d + 3 d F E_active)."""
    peak = (PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS) * 1e12
    F_alg = 2.0 * w.T * w.d * w.E + 6.0 * w.d * w.F * N
    B_alg = w.elt_bytes * (2.0 * w.T * w.d + w.E * w.d + 3.0 * w.d * w.F * E_active)
    return round(max(F_alg / peak, B_alg / (PEAK_HBM_GBS * 1e9)) / (ms * 1e-3), 4)


def device_inputs(w):
    import torch

    import moe_inputs as mi

    dev = {n: mi.device_tensor(w, n) for n in ("x", "w_router", "w_gate", "w_up", "w_down")}
    b_np = mi.router_bias(w)
    bias = None if b_np is None else torch.from_numpy(b_np).cuda()
    return (dev["x"], dev["w_router"], bias, dev["w_gate"], dev["w_up"], dev["w_down"])


def time_steps(run_step, K, stream):
    """Exactly K steps between synchronisations, an event after each: (ms/step, per-step ms,
    wall seconds)."""
    import torch

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(K):
        run_step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(K)]
    return ev[0].elapsed_time(ev[K]) / K, step_ms, wall


def staged_ms(lay, args_l, passes, stream) -> dict:
    """Mean ms of each stage of the layer run as its ABI calls with events between them.

    Each stage is its own ABI call from Python, and a short stage (the router, the
    dispatch) can finish on the GPU before the host has enqueued the next one.  The staged
    layers are therefore enqueued back to back with one synchronisation at the end: the host
    enqueues a layer's short stages while the GPU runs the previous layer's GEMMs, so the
    events time GPU work, not host gaps.  The first layer, which has no predecessor to hide
    behind, is not counted."""
    import torch

    runs = []
    for _ in range(passes + 1):
        e0 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        marks = []
        for name in lay.stages(*args_l):
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            marks.append((name, e))
        runs.append((e0, marks))
    torch.cuda.synchronize()
    times = {}
    for e0, marks in runs[1:]:
        prev = e0
        for name, e in marks:
            times.setdefault(name, []).append(prev.elapsed_time(e))
            prev = e
    return {n: statistics.mean(v) for n, v in times.items()}


SENTINEL = 0xA5


def written_extent(region_bytes) -> int:
    """Bytes from the start of a region to its last byte that no longer holds the sentinel
    (every region is written from its start: rows 0 .. N-1, tables, counters)."""
    import torch

    n = region_bytes.numel()
    if n == 0:
        return 0
    chunk = 1 << 16
    full = n // chunk * chunk
    last = -1
    if full:
        hit = (region_bytes[:full].view(-1, chunk) != SENTINEL).any(dim=1)
        nz = torch.nonzero(hit)
        if nz.numel():
            c = int(nz[-1])
            inner = torch.nonzero(region_bytes[c * chunk:(c + 1) * chunk] != SENTINEL)
            last = c * chunk + int(inner[-1])
    tail = torch.nonzero(region_bytes[full:] != SENTINEL)
    if tail.numel():
        last = full + int(tail[-1])
    return last + 1


def memory_by_phase(lay, args_l, moe) -> dict:
    """[EP-checks] "Memory must be counted by phase": the workspace bytes the layer has
    written by the end of each phase, measured (the workspace is filled with a sentinel
    byte, the layer runs stage by stage, and after each phase every region's written extent
    is read back) beside the library's bound (moe_workspace_phases), plus torch's allocated
    and peak figures.  The library allocates nothing, so torch's figures are flat across
    the phases: inputs, weights, outputs and the one workspace, allocated beforehand."""
    import torch

    s, ws = lay.shape, lay.workspace
    lay_off = moe.workspace_layout(s)
    names = moe.WS_REGIONS
    ends = [lay_off[names[i + 1]] if i + 1 < len(names) else ws.numel()
            for i in range(len(names))]
    ws.fill_(SENTINEL)
    torch.cuda.synchronize()

    def touched():
        per = {n: written_extent(ws[lay_off[n]:ends[i]]) for i, n in enumerate(names)}
        return sum(per.values()), per

    phase_of = {"dispatch": "after_pack", "down": "after_experts"}
    measured = {"before_layer": 0}
    alloc = {"before_layer": torch.cuda.memory_allocated()}
    per_region = {}
    for name in lay.stages(*args_l):
        if name in phase_of:
            torch.cuda.synchronize()
            total, per_region = touched()
            measured[phase_of[name]] = total
            alloc[phase_of[name]] = torch.cuda.memory_allocated()
    measured["after_dispatch"] = measured["after_pack"]  # expert-parallel size 1
    alloc["after_dispatch"] = alloc["after_pack"]
    bound = moe.workspace_phases(s)
    order = moe.PHASES
    return {
        "workspace_bytes": int(ws.numel()),
        "written_bytes_measured": {p: int(measured[p]) for p in order},
        "written_bytes_bound": {p: int(bound[p]) for p in order},
        "written_by_region_after_experts": {n: v for n, v in per_region.items() if v},
        "torch_allocated_bytes": {p: int(alloc[p]) for p in order},
        "torch_peak_allocated_bytes": int(torch.cuda.max_memory_allocated()),
        "torch_peak_reserved_bytes": int(torch.cuda.max_memory_reserved()),
    }


def routing_summary(moe, w, s, lay, ep, ranks_per_node) -> dict:
    """The layer's S9 record (moe_expert_stats over the routed and kept counts), drops, and
    the per-slot and placement record of moe_slot_counts' tables under a contiguous
    placement of the experts over `ep` ranks."""
    import numpy as np
    import torch

    routed = lay.routed_counts.cpu().numpy()
    kept = lay.tokens_per_expert.cpu().numpy()
    drops = lay.drops.cpu().numpy().astype(np.int64)
    rec = moe.expert_stats(w.T, w.k, routed, kept)
    stats = {"active_tokens": w.T, "top_k": w.k, "capacity": int(s.capacity),
             "expert_p50": rec["expert_p50"], "expert_p95": rec["expert_p95"],
             "expert_max": rec["expert_max"],
             "expert_max_to_mean": round(rec["expert_max_to_mean"], 4),
             "top_5_percent_expert_share": round(rec["top_5_percent_expert_share"], 4),
             "dropped_tokens": int(drops[0]), "dropped_per_slot": drops[1:w.k + 1].tolist(),
             "fully_dropped_tokens": int(drops[w.k + 1]), "kept_rows": rec["kept_rows"],
             "active_experts": rec["active_experts"]}
    if w.segments:
        stats["segments"] = segment_drops(lay.view("dest_row").cpu().numpy(), w.segments)
    rbs = torch.empty((w.k, w.E), dtype=torch.int32, device="cuda")
    kbs = torch.empty_like(rbs)
    moe.slot_counts(s, lay.view("topk_idx"), lay.view("dest_row"), rbs, kbs)
    placement = np.arange(w.E) * ep // w.E
    rr = moe.routing_record(w.T, rbs.cpu().numpy(), kbs.cpu().numpy(), placement,
                            ranks_per_node)
    stats["routing"] = {
        "slot_max_to_mean": [round(v, 3) for v in rr["slot_max_to_mean"]],
        "drop_share_per_slot": [round(v, 4) for v in rr["drop_share_per_slot"]],
        "ep_ranks": ep, "rank_load": rr["rank_load"],
        "rank_max_to_mean": round(rr["rank_max_to_mean"], 4),
        "node_load": rr["node_load"], "node_max_to_mean": round(rr["node_max_to_mean"], 4)}
    return stats


def measure(moe, w, s, args_l, K, W, graph=False, passes=5, ep=8, ranks_per_node=8,
            phases=True) -> dict:
    """Time K moe_layer steps of shape s after W warm-up steps, then the staged pass, the
    routing record, the rooflines and (phases) the memory record."""
    import torch

    lay = moe.MoELayer(s)
    stream = torch.cuda.current_stream()
    for _ in range(W):
        lay(*args_l)
    torch.cuda.synchronize()
    run_step = lambda: lay(*args_l)  # noqa: E731
    if graph:  # the same launches, replayed from a captured HIP graph
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            lay(*args_l)
        run_step = g.replay
        for _ in range(W):
            run_step()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
    ms, step_ms, wall = time_steps(run_step, K, stream)
    st = staged_ms(lay, args_l, max(K, passes), stream)
    stats = routing_summary(moe, w, s, lay, ep, ranks_per_node)
    N, E_active = stats["kept_rows"], stats["active_experts"]
    roof = gate_up_roofline(w, N, E_active, st["gate_up"])
    roof["traffic"] = traffic_for(w.name)
    roof["kernel"] = "prefill_gemm_kernel (gate/up + SwiGLU), incl. its tile-table launch"
    roof["kernel_ms"] = round(st["gate_up"], 4)
    out = {
        "ms_per_step": round(ms, 4), "tokens_per_s": round(w.T / (ms * 1e-3), 1),
        "wall_ms_per_step": round(wall * 1e3 / K, 4),
        "step_ms_p50_p95_p99": [round(percentile(step_ms, q), 4) for q in (0.5, 0.95, 0.99)],
        "roofline": roof,
        "down_roofline_frac": gate_up_roofline(w, N, E_active, 2.0 * st["down"])["frac"],
        "layer_roofline_frac": layer_roofline_frac(w, N, E_active, ms),
        "stage_ms": {"router_ms": round(st["router"], 4), "pack_ms": round(st["dispatch"], 4),
                     "expert_compute_ms": round(st["gate_up"] + st["down"], 4),
                     "gate_up_ms": round(st["gate_up"], 4), "down_ms": round(st["down"], 4),
                     "unpack_ms": round(st["combine"], 4)},
        "expert_stats": stats,
    }
    if phases:
        out["memory_by_phase"] = memory_by_phase(lay, args_l, moe)
    del lay
    return out


def cf_sweep(moe, w, args_l, factors, K, W, dtype) -> list:
    """[EP-checks] "Capacity factor changes quality, memory and tail latency": the same
    inputs at each capacity factor: drop rate per layer and per slot, step time p50 / p95 /
    p99, max over mean, and the workspace the capacity implies."""
    import torch

    rows = []
    for cf in factors:
        C = moe.capacity(w.T, w.k, w.E, cf)
        s = moe.shape(w.T, w.d, w.E, w.k, w.F, C, dtype)
        lay = moe.MoELayer(s)
        for _ in range(W):
            lay(*args_l)
        ms, step_ms, _ = time_steps(lambda: lay(*args_l), K, torch.cuda.current_stream())
        drops = lay.drops.cpu().numpy()
        rec = moe.expert_stats(w.T, w.k, lay.routed_counts.cpu().numpy(),
                               lay.tokens_per_expert.cpu().numpy())
        kept = lay.tokens_per_expert.cpu().numpy()
        rows.append({
            "capacity_factor": cf, "capacity": C,
            "drop_rate": round(float(drops[0]) / (w.T * w.k), 5),
            "drop_rate_per_slot": [round(float(v) / w.T, 5) for v in drops[1:w.k + 1]],
            "fully_dropped_tokens": int(drops[w.k + 1]),
            "ms_per_step": round(ms, 4),
            "step_ms_p50_p95_p99": [round(percentile(step_ms, q), 4) for q in (0.5, 0.95, 0.99)],
            "expert_max_to_mean": round(rec["expert_max_to_mean"], 4),
            "kept_max_to_mean": round(float(kept.max()) / (float(kept.sum()) / w.E), 4),
            "workspace_bytes": moe.workspace_size(s),
            "max_rows": moe.max_rows(s),
        })
        del lay
    return rows


def vendor_reference(w, N, reps=10) -> dict:
    """Reference points on the same GPU, outside the layer: hipBLASLt (through torch.matmul,
    plain 2-D products of contiguous bf16 operands) on the dense equivalents of the two
    grouped GEMMs (all N kept rows against one expert-sized weight, an easier shape than
    the grouped one), and a 1 GiB device-to-device copy as the attainable HBM rate."""
    import torch

    out = {}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    g = torch.Generator(device="cuda").manual_seed(5)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    for name, (m, kk, n) in (("gate_up", (N, w.d, 2 * w.F)), ("down", (N, w.F, w.d))):
        a = torch.randn((m, kk), generator=g, device="cuda").to(dt)
        b = (torch.randn((kk, n), generator=g, device="cuda") / math.sqrt(kk)).to(dt)
        ms = timed(lambda: torch.matmul(a, b))
        tf = 2.0 * m * kk * n / (ms * 1e-3) / 1e12
        out[f"dense_{name}"] = {"shape_mkn": [m, kk, n], "ms": round(ms, 4),
                                "tflops": round(tf, 1), "frac": round(tf / peak, 4)}
        del a, b
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = timed(lambda: dst.copy_(src))
    out["copy_1gib"] = {"ms": round(ms, 4), "gbs": round(2.0 * (1 << 30) / (ms * 1e-3) / 1e9, 1),
                        "frac_of_8tbs": round(2.0 * (1 << 30) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del src, dst
    torch.cuda.empty_cache()
    return out


class PowerSampler:
    """Socket power and graphics clock of this GPU from the driver's metrics table (amdsmi
    getters only; nothing is set), polled in a background thread.  The driver refreshes
    the table about once a second, so each phase loops its work for several seconds and is
    summarised over the refreshes that fall inside it."""

    def __init__(self):
        import threading

        import amdsmi
        import torch

        self.smi = amdsmi
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        props = torch.cuda.get_device_properties(torch.cuda.current_device())
        want = "%04x:%02x:%02x" % (getattr(props, "pci_domain_id", 0),
                                   getattr(props, "pci_bus_id", 0),
                                   getattr(props, "pci_device_id", 0))
        match = [h for h in handles
                 if str(amdsmi.amdsmi_get_gpu_device_bdf(h)).lower().startswith(want)]
        if not match and len(handles) != 1:
            raise RuntimeError(f"no metrics handle for the GPU at {want}")
        self.h = (match or handles)[0]
        self.cap_w = amdsmi.amdsmi_get_power_cap_info(self.h)["power_cap"] / 1e6
        self.samples, self.marks = [], []
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)
        self._t.start()

    def _run(self):
        while not self._stop.is_set():
            try:
                m = self.smi.amdsmi_get_gpu_metrics_info(self.h)
                clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int)]
                if not clks and isinstance(m.get("current_gfxclk"), int):
                    clks = [m["current_gfxclk"]]
                self.samples.append((time.time(), m.get("current_socket_power"),
                                     statistics.mean(clks) if clks else None,
                                     m.get("temperature_hotspot")))
            except Exception:  # noqa: BLE001  (a missed poll is retried)
                pass
            time.sleep(0.02)

    def phase(self, name, work, seconds):
        """Run work() (which enqueues a batch and synchronises) until `seconds` have passed."""
        t0 = time.time()
        while time.time() - t0 < seconds:
            work()
        self.marks.append((name, t0, time.time()))

    def close(self) -> dict:
        self._stop.set()
        self._t.join(timeout=5.0)  # a poll stuck in the driver must not hold the run
        if not self._t.is_alive():
            try:
                self.smi.amdsmi_shut_down()
            except Exception:  # noqa: BLE001  (the record is complete either way)
                pass
        return summarize_power(list(self.samples), self.marks, self.cap_w)


def summarize_power(samples, marks, cap_w) -> dict:
    """Per phase (name, t0, t1) of marks: the median socket power and graphics clock over the
    metric-table refreshes inside it.  samples: (time, power W, clock MHz, hotspot C) polls;
    consecutive polls that read the same power and clock are one refresh.  The first second
    of a phase is skipped: the table read then may still describe the time before it."""
    out = {"power_cap_w": cap_w, "source": "amdsmi gpu metrics (refreshed about once a second)"}
    for name, t0, t1 in marks:
        rows, prev = [], None
        for s in samples:
            if t0 + 1.1 <= s[0] <= t1 and (s[1], s[2]) != prev:
                rows.append(s)
                prev = (s[1], s[2])
        pw = [r[1] for r in rows if isinstance(r[1], (int, float))]
        ck = [r[2] for r in rows if isinstance(r[2], (int, float))]
        tp = [r[3] for r in rows if isinstance(r[3], (int, float))]
        p = statistics.median(pw) if pw else None
        out[name] = {"seconds": round(t1 - t0, 2), "refreshes": len(rows),
                     "socket_power_w": p,
                     "frac_of_cap": round(p / cap_w, 3) if p is not None and cap_w else None,
                     "gfx_clock_mhz": round(statistics.median(ck)) if ck else None,
                     "hotspot_c_max": max(tp) if tp else None}
    return out


def power_clock(moe, w, s, args_l, decode=None) -> dict:
    """Socket power and graphics clock: idle, the layer of shape s looped, the 16x16x32 MFMA
    calibration loop on random operands, and (decode = (shape, args)) an HBM-bound layer."""
    import torch

    ps = PowerSampler()
    ps.phase("idle", lambda: time.sleep(0.1), 2.5)
    lay = moe.MoELayer(s)

    def layer_batch(lay=lay, a=args_l):
        for _ in range(50):
            lay(*a)
        torch.cuda.synchronize()

    ps.phase(f"layer {w.name}", layer_batch, 5.0)
    del lay
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(cus * 8, dtype=torch.float32, device="cuda")
    cyc = torch.zeros(2 * cus, dtype=torch.int64, device="cuda")

    def calib_batch():
        for r in range(10):
            moe.calib_mfma(cus, 300_000, 2000 + r, True, sink, cyc, shape=1)
        torch.cuda.synchronize()

    ps.phase("mfma calibration loop, 16x16x32 random", calib_batch, 4.0)
    if decode is not None:
        lay_d = moe.MoELayer(decode[0])

        def decode_batch():
            for _ in range(50):
                lay_d(*decode[1])
            torch.cuda.synchronize()

        ps.phase("layer dsv3_decode", decode_batch, 4.0)
        del lay_d
    return ps.close()


def mfma_ceiling(moe, iters=300_000, reps=5, operands=("random", "zero")) -> dict:
    """The bf16 MFMA rate this GPU sustains with every SIMD of every CU issuing nothing but
    independent 32x32x16 MFMAs on register operands (libmoe_calib.so), and the shader clock
    it holds meanwhile (cycle counter over the constant-rate wall clock), for random operands
    (the data statistics of the layer) and for all-zero operands; and, for comparison, the
    16x16x32 form on random operands.  The published peak assumes
    the full clock; under this load the power limit sets the clock, so the random-operand
    rate is the ceiling an MFMA-bound kernel can approach."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(cus * 8, dtype=torch.float32, device="cuda")
    cyc = torch.zeros(2 * cus, dtype=torch.int64, device="cuda")
    khz = moe.calib_wall_clock_khz()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    out = {"cus": cus, "iters": iters}
    # 32x32x16 on random and on zero operands; 16x16x32 on random operands for comparison
    for label, rnd, shape in (("random_bf16", True, 0), ("zero_operands", False, 0),
                              ("random_bf16_16x16x32", True, 1)):
        if ("random" if rnd else "zero") not in operands:
            continue
        flops = cus * 8 * iters * 4 * (32768 if shape == 0 else 16384)
        for r in range(2):  # warm-up: the clock settles under the load
            moe.calib_mfma(cus, iters, 977 + r, rnd, sink, cyc, shape=shape)
        torch.cuda.synchronize()
        ms, ghz = [], []
        for r in range(reps):
            ev[0].record()
            moe.calib_mfma(cus, iters, 1000 + r, rnd, sink, cyc, shape=shape)
            ev[1].record()
            torch.cuda.synchronize()
            ms.append(ev[0].elapsed_time(ev[1]))
            c = cyc.view(cus, 2).sum(dim=0).tolist()
            ghz.append(c[0] / c[1] * khz * 1e3 / 1e9 if c[1] > 0 else float("nan"))
        assert bool(torch.isfinite(sink).all()), "calibration accumulators not finite"
        t = statistics.median(ms)
        tf = flops / (t * 1e-3) / 1e12
        out[label] = {"flops_per_launch": flops, "ms": round(t, 3), "tflops": round(tf, 1),
                      "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                      "clock_ghz": round(statistics.median(ghz), 3)}
    return out


OTHER_WORKLOADS = ["tiny_f32", "mixtral_8x22b_zipf", "dsv3_decode", "dsv3_mixed"]
SWEEP_WORKLOAD, SWEEP_FACTORS = "mixtral_8x22b_zipf", (1.0, 1.25, 1.5, 2.0, None)


def main():
    args = parse()
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters), indent=1))
        return
    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace), indent=1))
        return
    if args.summarize_traffic:
        t = summarize_traffic(*args.summarize_traffic, args.workload)
        path = os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json")
        json.dump(t, open(path, "w"), indent=1)
        print(json.dumps(t))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the MoE layer (expert parallel size 1); "
              "it does not run on several GPUs.", file=sys.stderr)
        sys.exit(2)
    build_if_missing()
    import torch

    import moe_inputs as mi
    import routing_expert_ffn_router_amd as moe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.mfma_ceiling:  # the calibration alone (for a counter run of it)
        ops = {"both": ("random", "zero"), "random": ("random",), "zero": ("zero",)}
        print(json.dumps({"mfma_ceiling": mfma_ceiling(moe, operands=ops[args.mfma_ceiling])}),
              flush=True)
        return
    if args.power:  # the power and clock record alone
        w = mi.WORKLOADS[DEFAULT_WORKLOAD]
        s = moe.shape(w.T, w.d, w.E, w.k, w.F, moe.capacity(w.T, w.k, w.E, w.capacity_factor),
                      moe.MOE_BF16)
        wd = mi.WORKLOADS["dsv3_decode"]
        sd = moe.shape(wd.T, wd.d, wd.E, wd.k, wd.F,
                       moe.capacity(wd.T, wd.k, wd.E, wd.capacity_factor), moe.MOE_BF16)
        rec = power_clock(moe, w, s, device_inputs(w), decode=(sd, device_inputs(wd)))
        print(json.dumps({"power_clock": rec}), flush=True)
        return
    w = mi.WORKLOADS[args.workload]
    cf = w.capacity_factor if args.capacity_factor is None else (
        None if args.capacity_factor <= 0 else args.capacity_factor)
    C = moe.capacity(w.T, w.k, w.E, cf)
    dtype = moe.MOE_BF16 if w.dtype == "bf16" else moe.MOE_F32
    flags = ((moe.MOE_FLAG_PAD_TO_CAPACITY if args.pad else 0) |
             (moe.MOE_FLAG_SLOT_MAJOR if args.slot_major else 0) |
             (moe.MOE_FLAG_BIAS_SELECTION_ONLY if args.bias_selection_only else 0))
    G, M = (int(v) for v in args.groups.split(":")) if args.groups else (0, 0)
    s = moe.shape(w.T, w.d, w.E, w.k, w.F, C, dtype, flags=flags, n_groups=G, topk_groups=M)
    print(f"# workload {w.name}: {s}", file=sys.stderr, flush=True)

    torch.cuda.reset_peak_memory_stats()
    args_l = device_inputs(w)
    m = measure(moe, w, s, args_l, args.steps, args.warmup, graph=args.graph, ep=args.ep,
                ranks_per_node=args.ranks_per_node)
    print(f"# timed {args.steps} steps: {m['ms_per_step']:.4f} ms/step "
          f"(wall {m['wall_ms_per_step']:.4f})", file=sys.stderr, flush=True)
    if args.copy_calibration:  # a plain device copy of known size, for counter scaling
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    sweep = None
    if args.cf_sweep:
        factors = [None if v in ("none", "0") else float(v) for v in args.cf_sweep.split(",")]
        sweep = cf_sweep(moe, w, args_l, factors, args.steps, args.warmup, dtype)
    del args_l
    torch.cuda.empty_cache()

    result = {
        "metric": METRIC,
        "value": m["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Philox inputs, random-init weights)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "E": w.E, "k": w.k, "F": w.F,
                   "capacity_factor": cf, "capacity": C,
                   "router_bias_zipf_s": w.zipf_s,
                   "dispatch": "pad_to_capacity" if args.pad else "packed",
                   "drop_order": "slot_major" if args.slot_major else "token_major",
                   "bias": "selection_only" if args.bias_selection_only else "logits",
                   "groups": [G, M] if G > 1 else None,
                   "launch": "hip_graph_replay" if args.graph else "stream"},
        "roofline": m["roofline"],
        "layer_roofline_frac": m["layer_roofline_frac"],
        "down_roofline_frac": m["down_roofline_frac"],
        "step_ms_p50_p95_p99": m["step_ms_p50_p95_p99"],
        "stage_ms": m["stage_ms"],
        "expert_stats": m["expert_stats"],
        "memory_by_phase": m["memory_by_phase"],
        "cpu_baseline": None,
    }
    if sweep is not None:
        result["cf_sweep"] = sweep
    # (a counter run with --copy-calibration keeps to the layer and the calibration copies:
    # the vendor reference's own device copy would be taken for one of them)
    default_run = not (flags or G > 1 or args.graph or args.capacity_factor is not None or
                       args.cf_sweep or args.workload != DEFAULT_WORKLOAD or
                       args.copy_calibration)
    if default_run:
        print("# vendor reference: hipBLASLt dense GEMMs, device copy", file=sys.stderr,
              flush=True)
        result["vendor_reference"] = vendor_reference(w, m["expert_stats"]["kept_rows"])
    if default_run and not args.no_other_workloads:
        # every other workload, timed the same way (fewer steps), and the capacity-factor
        # sweep of the skewed Mixtral-8x22B layer; reported beside the headline, not in it
        others = {}
        for name in OTHER_WORKLOADS:
            wo = mi.WORKLOADS[name]
            so = moe.shape(wo.T, wo.d, wo.E, wo.k, wo.F,
                           moe.capacity(wo.T, wo.k, wo.E, wo.capacity_factor),
                           moe.MOE_BF16 if wo.dtype == "bf16" else moe.MOE_F32)
            print(f"# workload {name}", file=sys.stderr, flush=True)
            al = device_inputs(wo)
            mo = measure(moe, wo, so, al, args.other_steps, args.warmup, phases=True)
            mo["config"] = {"T": wo.T, "d": wo.d, "E": wo.E, "k": wo.k, "F": wo.F,
                            "capacity_factor": wo.capacity_factor, "capacity": int(so.capacity),
                            "router_bias_zipf_s": wo.zipf_s, "dtype": wo.dtype}
            if name == SWEEP_WORKLOAD:
                print(f"# capacity-factor sweep on {name}", file=sys.stderr, flush=True)
                result["cf_sweep"] = {"workload": name, "rows": cf_sweep(
                    moe, wo, al, SWEEP_FACTORS, args.other_steps, args.warmup, moe.MOE_BF16)}
            others[name] = mo
            del al
            torch.cuda.empty_cache()
        result["workloads"] = others
    if default_run:
        print("# bf16 MFMA ceiling: register-operand MFMA loop on every SIMD", file=sys.stderr,
              flush=True)
        ceil = mfma_ceiling(moe)
        result["mfma_ceiling"] = ceil
        # the MFMA-bound GEMMs against the rate the chip sustains under the power limit with
        # the MFMA form they issue (16x16x32 in every bf16 prefill tile)
        top = ceil["random_bf16_16x16x32"]["tflops"]
        for roof in [result["roofline"]] + [v["roofline"] for v in
                                            result.get("workloads", {}).values()]:
            if roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == \
                    PEAK_BF16_TFLOPS:
                roof["frac_of_mfma_ceiling"] = round(roof["achieved"] / top, 4)
                roof["mfma_ceiling_form"] = "16x16x32"
        # socket power and graphics clock while the headline layer and the calibration loop
        # run (driver metrics): whether the power cap sets the clock
        print("# power and clock record", file=sys.stderr, flush=True)
        try:
            result["power_clock"] = power_clock(moe, w, s, device_inputs(w))
        except Exception as e:  # noqa: BLE001  (the record is optional, the run is not)
            result["power_clock"] = {"error": f"{type(e).__name__}: {e}"}
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline and not (flags or G > 1):
        ntok = args.cpu_tokens or CPU_SAMPLE_TOKENS.get(w.name, 256)
        print(f"# cpu baseline: oracle on {ntok} tokens", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, ntok)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
