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
sample of the same workload, is reported as a baseline.
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
    p.add_argument("--ep", type=int, default=8,
                   help="ranks of the expert placement in the routing record (contiguous)")
    p.add_argument("--ranks-per-node", type=int, default=8)
    p.add_argument("--graph", action="store_true",
                   help="time replays of a HIP graph that captured one moe_layer call")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a device copy of known size (for rocprofv3 --pmc scaling)")
    p.add_argument("--summarize-counters", metavar="PMC_DIR",
                   help="per kernel of a rocprofv3 --pmc ... --kernel-trace run: shader clock "
                        "(GRBM_COUNT), MFMA busy share (SQ_VALU_MFMA_BUSY_CYCLES over "
                        "GRBM_GUI_ACTIVE) and bf16 MFMA flops (SQ_INSTS_VALU_MFMA_MOPS_BF16), "
                        "for whichever of these counters the run holds")
    p.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                        "script into profiles/traffic_<workload>.json and exit")
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


def summarize_traffic(fetch_dir, write_dir, workload):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the dominant kernel, scaled by what the
    same counters read for the calibration copy of COPY_BYTES."""
    import statistics as st

    out = {"workload": workload, "kernel_source_sha": kernel_source_sha(),
           "copy_bytes": COPY_BYTES}
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
        mfma_tflops   = 512 * SQ_INSTS_VALU_MFMA_MOPS_BF16 / duration."""
    import csv
    import glob
    import re
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

    def short(name):
        if "prefill_gemm_kernel" in name:
            # bf16 operands with an fp32 output: the router logits in dense mode
            # (mangled: the output type f, possibly followed by a back-reference, closes the
            # template arguments; demangled: ", float" among them)
            if ("IDF16b" in name and re.search(r"f(?:S\d*_)?EEvPKT_", name)) or (
                    "__bf16" in name and re.search(r", float[,>]", name)):
                return "prefill_gemm_kernel (router logits, dense)"
            return "prefill_gemm_kernel (" + (
                "down" if "Lb0E" in name or "false" in name else "gate/up+SwiGLU") + ")"
        return name.split("(")[0].split("<")[0].replace("void ", "")

    per = {}
    for e in disp.values():
        ns = e["ns"]
        f = {"ns": ns}
        if "GRBM_COUNT" in e:
            f["clock_ghz"] = e["GRBM_COUNT"] / n_xcc / ns
        if "SQ_VALU_MFMA_BUSY_CYCLES" in e and e.get("GRBM_GUI_ACTIVE"):
            f["mfma_busy_pct"] = (100.0 * e["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                  (e["GRBM_GUI_ACTIVE"] / n_xcc * n_simd))
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in e:
            f["mfma_tflops"] = 512.0 * e["SQ_INSTS_VALU_MFMA_MOPS_BF16"] / ns / 1e3
            f["mfma_gflop_per_dispatch"] = 512.0 * e["SQ_INSTS_VALU_MFMA_MOPS_BF16"] / 1e9
        per.setdefault(short(e["name"]), []).append(f)
    out = []
    for name, v in sorted(per.items(), key=lambda kv: -sum(f["ns"] for f in kv[1])):
        k = {"kernel": name, "dispatches": len(v),
             "median_us": round(st.median(f["ns"] for f in v) / 1e3, 1)}
        for key, nd in (("clock_ghz", 3), ("mfma_busy_pct", 1), ("mfma_tflops", 1),
                        ("mfma_gflop_per_dispatch", 2)):
            vals = [f[key] for f in v if key in f]
            if vals:
                k[key] = round(st.median(vals), nd)
        out.append(k)
    return {"xcds": n_xcc, "simds": n_simd, "kernels": out}


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
    recomputed for ntok tokens with the same factor), full router and expert weights."""
    import numpy as np
    import threadpoolctl

    import moe_inputs as mi
    import oracle

    x = mi.host_tensor_f32(w, "x", 0, ntok)
    wr = mi.host_tensor_f32(w, "w_router")
    b = mi.router_bias(w)
    wg, wu, wd = (mi.host_tensor_f32(w, n) for n in ("w_gate", "w_up", "w_down"))
    C = oracle.capacity(ntok, w.k, w.E, w.capacity_factor)
    t0 = time.perf_counter()
    res = oracle.moe_layer(x, wr, b, wg, wu, wd, w.k, C)
    dt = time.perf_counter() - t0
    assert np.all(np.isfinite(res["out"]))
    threads = 0
    for info in threadpoolctl.threadpool_info():
        threads = max(threads, int(info.get("num_threads", 0)))
    return {"value": ntok / dt, "unit": "tokens/s", "cores": threads or os.cpu_count(),
            "kind": "oracle", "seconds": round(dt, 3),
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


def main():
    args = parse()
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters), indent=1))
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
    import numpy as np
    import torch

    import moe_inputs as mi
    import routing_expert_ffn_router_amd as moe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = mi.WORKLOADS[args.workload]
    C = moe.capacity(w.T, w.k, w.E, w.capacity_factor)
    dtype = moe.MOE_BF16 if w.dtype == "bf16" else moe.MOE_F32
    flags = ((moe.MOE_FLAG_PAD_TO_CAPACITY if args.pad else 0) |
             (moe.MOE_FLAG_SLOT_MAJOR if args.slot_major else 0) |
             (moe.MOE_FLAG_BIAS_SELECTION_ONLY if args.bias_selection_only else 0))
    G, M = (int(v) for v in args.groups.split(":")) if args.groups else (0, 0)
    s = moe.shape(w.T, w.d, w.E, w.k, w.F, C, dtype, flags=flags, n_groups=G, topk_groups=M)
    b_elt = w.elt_bytes
    print(f"# workload {w.name}: {s}", file=sys.stderr, flush=True)

    dev = {n: mi.device_tensor(w, n) for n in ("x", "w_router", "w_gate", "w_up", "w_down")}
    b_np = mi.router_bias(w)
    bias = None if b_np is None else torch.from_numpy(b_np).cuda()
    args_l = (dev["x"], dev["w_router"], bias, dev["w_gate"], dev["w_up"], dev["w_down"])
    lay = moe.MoELayer(s)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        lay(*args_l)
    torch.cuda.synchronize()
    run_step = lambda: lay(*args_l)  # noqa: E731
    if args.graph:  # the same launches, replayed from a captured HIP graph
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            lay(*args_l)
        run_step = graph.replay
        for _ in range(args.warmup):
            run_step()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()

    # ---- timed region: exactly K moe_layer calls ------------------------------------------
    K = args.steps
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
    total_ms = ev[0].elapsed_time(ev[K])
    ms_per_step = total_ms / K
    print(f"# timed {K} steps: {ms_per_step:.4f} ms/step (wall {wall * 1e3 / K:.4f})",
          file=sys.stderr, flush=True)

    # ---- staged pass: the same launches with events between the ABI calls ------------------
    # Each stage is its own ABI call from Python, and a short stage (the router, the
    # dispatch) can finish on the GPU before the host has enqueued the next one.  The
    # staged layers are therefore enqueued back to back with one synchronisation at the
    # end: the host enqueues a layer's short stages while the GPU runs the previous layer's
    # GEMMs, so the events time GPU work, not host gaps.  The first layer, which has no
    # predecessor to hide behind, is not counted.
    stage_times = {}
    passes = []
    for i in range(max(K, 5) + 1):
        e0 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        marks = []
        for name in lay.stages(*args_l):
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            marks.append((name, e))
        passes.append((e0, marks))
    torch.cuda.synchronize()
    for e0, marks in passes[1:]:
        prev = e0
        for name, e in marks:
            stage_times.setdefault(name, []).append(prev.elapsed_time(e))
            prev = e
    stage_ms = {n: statistics.mean(v) for n, v in stage_times.items()}

    if args.copy_calibration:  # a plain device copy of known size, for counter scaling
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- routing statistics of the last call ------------------------------------------------
    routed = lay.routed_counts.cpu().numpy().astype(np.int64)
    kept = lay.tokens_per_expert.cpu().numpy().astype(np.int64)
    drops = lay.drops.cpu().numpy().astype(np.int64)
    rec = moe.expert_stats(w.T, w.k, routed, kept)  # the library's S9 record
    N = rec["kept_rows"]
    E_active = rec["active_experts"]
    stats = {"active_tokens": w.T, "top_k": w.k, "capacity": C,
             "expert_p50": rec["expert_p50"], "expert_p95": rec["expert_p95"],
             "expert_max": rec["expert_max"],
             "expert_max_to_mean": round(rec["expert_max_to_mean"], 4),
             "dropped_tokens": int(drops[0]), "dropped_per_slot": drops[1:w.k + 1].tolist(),
             "fully_dropped_tokens": int(drops[w.k + 1]), "kept_rows": N,
             "active_experts": E_active}
    if w.segments:
        stats["segments"] = segment_drops(lay.view("dest_row").cpu().numpy(), w.segments)
    if args.pad:
        R = moe.max_rows(s)
        stats["padded_rows"] = R
        stats["pad_fraction"] = round(1.0 - N / R, 4)
    # per-slot counts on the device, summarised on the host, under a contiguous placement of
    # the experts over --ep ranks
    rbs = torch.empty((w.k, w.E), dtype=torch.int32, device="cuda")
    kbs = torch.empty_like(rbs)
    moe.slot_counts(s, lay.view("topk_idx"), lay.view("dest_row"), rbs, kbs)
    placement = np.arange(w.E) * args.ep // w.E
    rec = moe.routing_record(w.T, rbs.cpu().numpy(), kbs.cpu().numpy(), placement,
                             args.ranks_per_node)
    stats["routing"] = {
        "top_5_percent_expert_share": round(rec["top_5_percent_expert_share"], 4),
        "slot_max_to_mean": [round(v, 3) for v in rec["slot_max_to_mean"]],
        "drop_share_per_slot": [round(v, 4) for v in rec["drop_share_per_slot"]],
        "ep_ranks": args.ep, "rank_load": rec["rank_load"],
        "rank_max_to_mean": round(rec["rank_max_to_mean"], 4),
        "node_load": rec["node_load"], "node_max_to_mean": round(rec["node_max_to_mean"], 4)}

    # ---- roofline of the dominant kernel (gate/up grouped GEMM) ------------------------------
    t_gu = stage_ms["gate_up"] * 1e-3
    flops_gu = 4.0 * N * w.d * w.F
    bytes_gu = b_elt * (2.0 * E_active * w.F * w.d + N * w.d + N * w.F)
    peak_flops = (PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS) * 1e12
    ridge = peak_flops / (PEAK_HBM_GBS * 1e9)
    if flops_gu / bytes_gu >= ridge:
        roof = {"bound": "mfma", "achieved": round(flops_gu / t_gu / 1e12, 2),
                "peak": peak_flops / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(bytes_gu / t_gu / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = traffic_for(w.name)
    roof["kernel"] = "prefill_gemm_kernel (gate/up + SwiGLU), incl. its tile-table launch"
    roof["kernel_ms"] = round(stage_ms["gate_up"], 4)

    # whole-layer roofline: algorithmic work of the layer against both peaks
    F_alg = 2.0 * w.T * w.d * w.E + 6.0 * w.d * w.F * N
    B_alg = b_elt * (2.0 * w.T * w.d + w.E * w.d + 3.0 * w.d * w.F * E_active)
    t_roof = max(F_alg / peak_flops, B_alg / (PEAK_HBM_GBS * 1e9))
    layer_frac = t_roof / (ms_per_step * 1e-3)

    result = {
        "metric": METRIC,
        "value": round(w.T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Philox inputs, random-init weights)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "E": w.E, "k": w.k, "F": w.F,
                   "capacity_factor": w.capacity_factor, "capacity": C,
                   "router_bias_zipf_s": w.zipf_s,
                   "dispatch": "pad_to_capacity" if args.pad else "packed",
                   "drop_order": "slot_major" if args.slot_major else "token_major",
                   "bias": "selection_only" if args.bias_selection_only else "logits",
                   "groups": [G, M] if G > 1 else None,
                   "launch": "hip_graph_replay" if args.graph else "stream"},
        "roofline": roof,
        "layer_roofline_frac": round(layer_frac, 4),
        "step_ms_p50_p95_p99": [round(percentile(step_ms, q), 4) for q in (0.5, 0.95, 0.99)],
        "stage_ms": {"router_ms": round(stage_ms["router"], 4),
                     "pack_ms": round(stage_ms["dispatch"], 4),
                     "expert_compute_ms": round(stage_ms["gate_up"] + stage_ms["down"], 4),
                     "gate_up_ms": round(stage_ms["gate_up"], 4),
                     "down_ms": round(stage_ms["down"], 4),
                     "unpack_ms": round(stage_ms["combine"], 4)},
        "expert_stats": stats,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and not (flags or G > 1):
        ntok = args.cpu_tokens or CPU_SAMPLE_TOKENS.get(w.name, 256)
        print(f"# cpu baseline: oracle on {ntok} tokens", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, ntok)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
