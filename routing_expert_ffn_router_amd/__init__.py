"""One GPU's share of a Mixture-of-Experts layer on MI355X (gfx950).

A thin ctypes binding of libmoe.so, whose C ABI is declared in include/moe.h.  The functions
here only marshal arguments (device pointers of torch tensors, the current HIP stream);
every step of the layer runs in the library's HIP kernels.  PyTorch provides device memory
and streams.  If libmoe.so is missing, loading fails with an error: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "moe.h")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_ALIGNMENT = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5
MOE_ERR_SCRATCH = -6
DISPATCH_SCRATCH_BYTES = 8 << 20  # MOE_DISPATCH_SCRATCH_BYTES

MOE_F32 = 0
MOE_BF16 = 1

MOE_FLAG_PAD_TO_CAPACITY = 1
MOE_FLAG_SLOT_MAJOR = 2
MOE_FLAG_BIAS_SELECTION_ONLY = 4

PHASES = ["before_layer", "after_pack", "after_dispatch", "after_experts"]

WS_REGIONS = ["logits", "topk_idx", "topk_w", "routed", "kept", "offsets", "src_token",
              "dest_row", "drops", "status", "tile_hist", "tile_base", "sched", "x_perm", "h",
              "y_perm", "down_acc"]


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("E", ctypes.c_int64),
                ("k", ctypes.c_int64), ("F", ctypes.c_int64), ("capacity", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32)]

    def __repr__(self):
        return (f"MoeShape(T={self.T}, d={self.d}, E={self.E}, k={self.k}, F={self.F}, "
                f"capacity={self.capacity}, dtype={'bf16' if self.dtype == 1 else 'f32'}, "
                f"flags={self.flags}, n_groups={self.n_groups}, "
                f"topk_groups={self.topk_groups})")


class ExpertStats(ctypes.Structure):
    """moe_expert_stats_t: the per-layer expert statistics record (see include/moe.h)."""
    _fields_ = [("active_tokens", ctypes.c_int64), ("top_k", ctypes.c_int64),
                ("experts", ctypes.c_int64), ("routed", ctypes.c_int64),
                ("expert_p50", ctypes.c_int64), ("expert_p95", ctypes.c_int64),
                ("expert_max", ctypes.c_int64), ("expert_mean", ctypes.c_double),
                ("expert_max_to_mean", ctypes.c_double),
                ("top_5_percent_experts", ctypes.c_int64),
                ("top_5_percent_expert_share", ctypes.c_double),
                ("kept_rows", ctypes.c_int64), ("active_experts", ctypes.c_int64),
                ("dropped_tokens", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


_lib = None
_P = ctypes.c_void_p
_S = ctypes.POINTER(MoeShape)


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    if path == LIB_PATH:
        from . import _build

        if not _build.is_current():
            raise RuntimeError(f"{path} was built from other sources than the ones in "
                               "csrc/ and include/; run __graft_entry__.build() again")
    # torch ships its own HIP runtime with the same soname as the system one; importing
    # torch first makes libmoe.so bind to that copy, so tensors, streams and kernels all
    # live in one runtime (two copies in one process break launches on torch's streams).
    import torch  # noqa: F401

    lib = ctypes.CDLL(path)
    i64, i32, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    sig = {
        "moe_capacity": (i64, [i64, i64, i64, ctypes.c_double]),
        "moe_max_rows": (i64, [_S]),
        "moe_workspace_size": (sz, [_S]),
        "moe_workspace_layout": (i32, [_S, ctypes.POINTER(i64)]),
        "moe_workspace_phases": (i32, [_S, ctypes.POINTER(i64)]),
        "moe_expert_stats": (i32, [i64, i64, i64, _P, _P, ctypes.POINTER(ExpertStats)]),
        "moe_slot_stats": (i32, [i64, i64, i64, _P, _P, _P, _P]),
        "moe_placement_load": (i32, [i64, _P, _P, i64, i64, _P, _P, _P]),
        "moe_status_string": (ctypes.c_char_p, [i32]),
        "moe_route": (i32, [_S, _P, _P, _P, _P, i32, _P, _P, _P, _P]),
        "moe_dispatch": (i32, [_S, _P, _P, _P, sz, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
        "moe_dispatch_no_workspace": (i32, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
        "moe_expert_ffn": (i32, [_S, _P, _P, _P, _P, _P, _P, sz, _P, _P]),
        "moe_expert_gate_up": (i32, [_S, _P, _P, _P, _P, _P, sz, _P, _P]),
        "moe_expert_gate_up_gathered": (i32, [_S, _P, _P, _P, _P, _P, _P, sz, _P, _P]),
        "moe_expert_down": (i32, [_S, _P, _P, _P, _P, sz, _P, _P]),
        "moe_combine": (i32, [_S, _P, _P, _P, _P, _P]),
        "moe_slot_counts": (i32, [_S, _P, _P, _P, _P, _P]),
        "moe_layer": (i32, [_S, _P, _P, _P, _P, _P, _P, _P, sz, _P, _P, _P, _P, _P, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions(path: str = HEADER_PATH) -> list:
    """Names of the functions include/moe.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()


def shape(T: int, d: int, E: int, k: int, F: int, capacity: int = 0,
          dtype: int = MOE_BF16, flags: int = 0, n_groups: int = 0,
          topk_groups: int = 0) -> MoeShape:
    return MoeShape(T, d, E, k, F, capacity, dtype, flags, n_groups, topk_groups)


def capacity(T: int, k: int, E: int, cf: Optional[float]) -> int:
    """Per-expert capacity of a capacity factor (0 = no limit); see moe_capacity."""
    return int(load_library().moe_capacity(T, k, E, 0.0 if cf is None else float(cf)))


def max_rows(s: MoeShape) -> int:
    return int(load_library().moe_max_rows(ctypes.byref(s)))


def workspace_size(s: MoeShape) -> int:
    return int(load_library().moe_workspace_size(ctypes.byref(s)))


def workspace_layout(s: MoeShape) -> dict:
    offs = (ctypes.c_int64 * len(WS_REGIONS))()
    rc = load_library().moe_workspace_layout(ctypes.byref(s), offs)
    if rc != MOE_OK:
        raise MoeError("moe_workspace_layout", rc)
    return {n: int(o) for n, o in zip(WS_REGIONS, offs)}


def workspace_phases(s: MoeShape) -> dict:
    """Workspace bytes moe_layer has written by the end of each phase (moe_workspace_phases)."""
    out = (ctypes.c_int64 * len(PHASES))()
    rc = load_library().moe_workspace_phases(ctypes.byref(s), out)
    if rc != MOE_OK:
        raise MoeError("moe_workspace_phases", rc)
    return {n: int(v) for n, v in zip(PHASES, out)}


def _host_i32(a):
    """A C-contiguous int32 numpy copy of a host array (or of a CPU tensor)."""
    import numpy as np

    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def expert_stats(T: int, k: int, routed_counts, tokens_per_expert=None) -> dict:
    """The per-layer expert statistics record (moe_expert_stats) of host count arrays."""
    n = _host_i32(routed_counts)
    c = None if tokens_per_expert is None else _host_i32(tokens_per_expert)
    if c is not None and c.shape != n.shape:
        raise ValueError("routed_counts and tokens_per_expert differ in length")
    rec = ExpertStats()
    _check("moe_expert_stats", load_library().moe_expert_stats(
        int(T), int(k), int(n.size), n.ctypes.data, None if c is None else c.ctypes.data,
        ctypes.byref(rec)))
    return rec.as_dict()


def slot_stats(T: int, routed_by_slot, kept_by_slot) -> dict:
    """moe_slot_stats of host [k, E] tables: each slot's max over mean and its share of the
    drops."""
    import numpy as np

    r, c = _host_i32(routed_by_slot), _host_i32(kept_by_slot)
    if r.ndim != 2 or r.shape != c.shape:
        raise ValueError("routed_by_slot and kept_by_slot must be [k, E] arrays")
    k, E = r.shape
    mtm, share = np.zeros(k), np.zeros(k)
    _check("moe_slot_stats", load_library().moe_slot_stats(
        int(T), k, E, r.ctypes.data, c.ctypes.data, mtm.ctypes.data, share.ctypes.data))
    return {"slot_max_to_mean": mtm.tolist(), "drop_share_per_slot": share.tolist()}


def placement_load(routed_counts, placement, n_ranks: int, ranks_per_node: int = 0) -> dict:
    """moe_placement_load: routed load per rank (and per node) under an expert placement."""
    import numpy as np

    n, pl = _host_i32(routed_counts), _host_i32(placement)
    if n.shape != pl.shape:
        raise ValueError("routed_counts and placement differ in length")
    nodes = -(-n_ranks // ranks_per_node) if ranks_per_node > 0 else 0
    rank_load = np.zeros(n_ranks, dtype=np.int64)
    node_load = np.zeros(max(nodes, 1), dtype=np.int64)
    mtm = np.zeros(2)
    _check("moe_placement_load", load_library().moe_placement_load(
        n.size, n.ctypes.data, pl.ctypes.data, int(n_ranks), int(ranks_per_node),
        rank_load.ctypes.data, node_load.ctypes.data if nodes else None, mtm.ctypes.data))
    out = {"rank_load": rank_load.tolist(), "rank_max_to_mean": float(mtm[0])}
    if nodes:
        out["node_load"] = node_load[:nodes].tolist()
        out["node_max_to_mean"] = float(mtm[1])
    return out


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check(fn: str, rc: int):
    if rc != MOE_OK:
        raise MoeError(fn, rc)


def route(s: MoeShape, x, w_router, b_router, logits, topk_idx, topk_w, status=None,
          logits_given: bool = False, stream=None) -> None:
    _check("moe_route", load_library().moe_route(
        ctypes.byref(s), _ptr(x), _ptr(w_router), _ptr(b_router), _ptr(logits),
        int(bool(logits_given)), _ptr(topk_idx), _ptr(topk_w), _ptr(status), _stream(stream)))


def dispatch(s: MoeShape, topk_idx, x, workspace, routed_counts, tokens_per_expert,
             expert_offsets, src_token, dest_row, drops, x_perm, stream=None,
             src_slot=None) -> None:
    _check("moe_dispatch", load_library().moe_dispatch(
        ctypes.byref(s), _ptr(topk_idx), _ptr(x), _ptr(workspace), _nbytes(workspace),
        _ptr(routed_counts), _ptr(tokens_per_expert), _ptr(expert_offsets), _ptr(src_token),
        _ptr(src_slot), _ptr(dest_row), _ptr(drops), _ptr(x_perm), _stream(stream)))


def dispatch_no_workspace(s: MoeShape, topk_idx, x, routed_counts, tokens_per_expert,
                          expert_offsets, src_token, dest_row, drops, x_perm, stream=None,
                          src_slot=None) -> None:
    """moe_dispatch without a workspace: its scratch tables live in the library's static
    per-GPU array (calls that overlap on one GPU race)."""
    _check("moe_dispatch_no_workspace", load_library().moe_dispatch_no_workspace(
        ctypes.byref(s), _ptr(topk_idx), _ptr(x), _ptr(routed_counts), _ptr(tokens_per_expert),
        _ptr(expert_offsets), _ptr(src_token), _ptr(src_slot), _ptr(dest_row), _ptr(drops),
        _ptr(x_perm), _stream(stream)))


def expert_ffn(s: MoeShape, x_perm, expert_offsets, w_gate, w_up, w_down, workspace, y_perm,
               stream=None) -> None:
    _check("moe_expert_ffn", load_library().moe_expert_ffn(
        ctypes.byref(s), _ptr(x_perm), _ptr(expert_offsets), _ptr(w_gate), _ptr(w_up),
        _ptr(w_down), _ptr(workspace), _nbytes(workspace), _ptr(y_perm), _stream(stream)))


def expert_gate_up(s: MoeShape, x_perm, expert_offsets, w_gate, w_up, workspace, h,
                   stream=None) -> None:
    _check("moe_expert_gate_up", load_library().moe_expert_gate_up(
        ctypes.byref(s), _ptr(x_perm), _ptr(expert_offsets), _ptr(w_gate), _ptr(w_up),
        _ptr(workspace), _nbytes(workspace), _ptr(h), _stream(stream)))


def expert_gate_up_gathered(s: MoeShape, x, src_token, expert_offsets, w_gate, w_up,
                            workspace, h, stream=None) -> None:
    _check("moe_expert_gate_up_gathered", load_library().moe_expert_gate_up_gathered(
        ctypes.byref(s), _ptr(x), _ptr(src_token), _ptr(expert_offsets), _ptr(w_gate),
        _ptr(w_up), _ptr(workspace), _nbytes(workspace), _ptr(h), _stream(stream)))


def gathered_layer(s: MoeShape) -> bool:
    """Whether moe_layer lets the gate/up GEMM gather the token rows (packed rows and x
    addressable with 32-bit offsets); x_perm is then not written."""
    esz = 2 if s.dtype == MOE_BF16 else 4
    return not (s.flags & MOE_FLAG_PAD_TO_CAPACITY) and s.T * s.d * esz < (1 << 31)


def expert_down(s: MoeShape, h, expert_offsets, w_down, workspace, y_perm,
                stream=None) -> None:
    _check("moe_expert_down", load_library().moe_expert_down(
        ctypes.byref(s), _ptr(h), _ptr(expert_offsets), _ptr(w_down), _ptr(workspace),
        _nbytes(workspace), _ptr(y_perm), _stream(stream)))


def combine(s: MoeShape, y_perm, dest_row, topk_w, out, stream=None) -> None:
    _check("moe_combine", load_library().moe_combine(
        ctypes.byref(s), _ptr(y_perm), _ptr(dest_row), _ptr(topk_w), _ptr(out),
        _stream(stream)))


def slot_counts(s: MoeShape, topk_idx, dest_row, routed_by_slot, kept_by_slot,
                stream=None) -> None:
    _check("moe_slot_counts", load_library().moe_slot_counts(
        ctypes.byref(s), _ptr(topk_idx), _ptr(dest_row), _ptr(routed_by_slot),
        _ptr(kept_by_slot), _stream(stream)))


def routing_record(T: int, routed_by_slot, kept_by_slot, placement=None,
                   ranks_per_node: Optional[int] = None) -> dict:
    """The observability record of moe_slot_counts' per-slot tables (host arrays [k, E]):
    the share of the busiest ceil(5 % of E) experts (moe_expert_stats), each slot's max over
    mean and share of the drops (moe_slot_stats) and, for an expert -> rank placement, the
    load per rank and per node (moe_placement_load)."""
    import numpy as np

    rbs, kbs = _host_i32(routed_by_slot), _host_i32(kept_by_slot)
    k = rbs.shape[0]
    n = rbs.sum(axis=0)
    st = expert_stats(T, k, n)
    rec = {"routed_by_slot": rbs.tolist(), "kept_by_slot": kbs.tolist(),
           "top_5_percent_experts": st["top_5_percent_experts"],
           "top_5_percent_expert_share": st["top_5_percent_expert_share"]}
    rec.update(slot_stats(T, rbs, kbs))
    if placement is not None:
        pl = np.asarray(placement)
        rec.update(placement_load(n, pl, int(pl.max()) + 1, int(ranks_per_node or 0)))
    return rec


def layer(s: MoeShape, x, w_router, b_router, w_gate, w_up, w_down, workspace, out,
          routed_counts=None, tokens_per_expert=None, drops=None, status=None,
          stream=None) -> None:
    _check("moe_layer", load_library().moe_layer(
        ctypes.byref(s), _ptr(x), _ptr(w_router), _ptr(b_router), _ptr(w_gate), _ptr(w_up),
        _ptr(w_down), _ptr(workspace), _nbytes(workspace), _ptr(out), _ptr(routed_counts),
        _ptr(tokens_per_expert), _ptr(drops), _ptr(status), _stream(stream)))


def workspace_view(workspace, s: MoeShape, region: str):
    """A typed view of one workspace region (for reading moe_layer's intermediate tables)."""
    import torch

    lay = workspace_layout(s)
    off = lay[region]
    T, E, k, d, F = s.T, s.E, s.k, s.d, s.F
    R = max_rows(s)
    act = torch.bfloat16 if s.dtype == MOE_BF16 else torch.float32
    spec = {
        "logits": (torch.float32, (T, E)), "topk_idx": (torch.int32, (T, k)),
        "topk_w": (torch.float32, (T, k)), "routed": (torch.int32, (E,)),
        "kept": (torch.int32, (E,)), "offsets": (torch.int32, (E + 1,)),
        "src_token": (torch.int32, (R,)), "dest_row": (torch.int32, (T, k)),
        "drops": (torch.int32, (k + 2,)), "status": (torch.int32, (1,)),
        "x_perm": (act, (R, d)), "h": (act, (R, F)), "y_perm": (act, (R, d)),
    }
    dt, shp = spec[region]
    n = 1
    for v in shp:
        n *= v
    esz = torch.tensor([], dtype=dt).element_size()
    return workspace[off:off + n * esz].view(dt).view(shp)


class MoELayer:
    """Convenience owner of the workspace and outputs of moe_layer for one shape."""

    def __init__(self, s: MoeShape, device="cuda"):
        import torch

        self.shape = s
        self.workspace = torch.empty(workspace_size(s), dtype=torch.uint8, device=device)
        act = torch.bfloat16 if s.dtype == MOE_BF16 else torch.float32
        self.out = torch.empty((s.T, s.d), dtype=act, device=device)
        self.routed_counts = torch.empty(s.E, dtype=torch.int32, device=device)
        self.tokens_per_expert = torch.empty(s.E, dtype=torch.int32, device=device)
        self.drops = torch.empty(s.k + 2, dtype=torch.int32, device=device)
        self.status = torch.empty(1, dtype=torch.int32, device=device)

    def __call__(self, x, w_router, b_router, w_gate, w_up, w_down, stream=None):
        layer(self.shape, x, w_router, b_router, w_gate, w_up, w_down, self.workspace,
              self.out, self.routed_counts, self.tokens_per_expert, self.drops, self.status,
              stream)
        return self.out

    def view(self, region: str):
        return workspace_view(self.workspace, self.shape, region)

    def stages(self, x, w_router, b_router, w_gate, w_up, w_down, stream=None):
        """The same layer as __call__, as five public ABI calls (route, dispatch, gate/up
        GEMM, down GEMM, combine; the dispatch builds the tables only and the gate/up GEMM
        gathers the rows when moe_layer does so), yielding after each one so a caller can
        record events between stages.  The same kernels run, except that moe_layer's
        dispatch also writes the GEMMs' tile table, which moe_expert_gate_up builds with a
        launch of its own here."""
        s, ws = self.shape, self.workspace
        v = self.view
        route(s, x, w_router, b_router, v("logits"), v("topk_idx"), v("topk_w"), self.status,
              stream=stream)
        yield "router"
        gathered = gathered_layer(s)
        dispatch(s, v("topk_idx"), x, ws, self.routed_counts, self.tokens_per_expert,
                 v("offsets"), v("src_token"), v("dest_row"), self.drops,
                 None if gathered else v("x_perm"), stream=stream)
        yield "dispatch"
        if gathered:
            expert_gate_up_gathered(s, x, v("src_token"), v("offsets"), w_gate, w_up, ws, v("h"),
                                    stream=stream)
        else:
            expert_gate_up(s, v("x_perm"), v("offsets"), w_gate, w_up, ws, v("h"),
                           stream=stream)
        yield "gate_up"
        expert_down(s, v("h"), v("offsets"), w_down, ws, v("y_perm"), stream=stream)
        yield "down"
        combine(s, v("y_perm"), v("dest_row"), v("topk_w"), self.out, stream=stream)
        yield "combine"


# ------------------------------------------------------------------------------ calibration
CALIB_PATH = os.path.join(_PKG, "libmoe_calib.so")
_calib = None


def load_calib() -> ctypes.CDLL:
    """Load libmoe_calib.so (include/moe_calib.h): the MFMA-rate calibration that the
    measurement harness reports beside the published peak.  Not part of the layer."""
    global _calib
    if _calib is None:
        load_library()  # the staleness check covers both libraries; binds torch's runtime
        lib = ctypes.CDLL(CALIB_PATH)
        lib.moe_calib_mfma.restype = ctypes.c_int
        lib.moe_calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_int,
                                       ctypes.c_int, _P, _P, _P]
        lib.moe_calib_wall_clock_khz.restype = ctypes.c_int
        lib.moe_calib_wall_clock_khz.argtypes = [ctypes.POINTER(ctypes.c_int)]
        _calib = lib
    return _calib


def calib_mfma(blocks: int, iters: int, seed: int, random_operands: bool, sink, cycles,
               shape: int = 0, stream=None) -> None:
    """Enqueue moe_calib_mfma (shape 0: 32x32x16, 1: 16x16x32): sink float32[blocks * 8],
    cycles int64[2 * blocks] on the GPU."""
    _check("moe_calib_mfma", load_calib().moe_calib_mfma(
        int(blocks), int(iters), int(seed) & 0xFFFFFFFF, int(bool(random_operands)), int(shape),
        _ptr(sink), _ptr(cycles), _stream(stream)))


def calib_wall_clock_khz() -> int:
    khz = ctypes.c_int(0)
    _check("moe_calib_wall_clock_khz", load_calib().moe_calib_wall_clock_khz(ctypes.byref(khz)))
    return int(khz.value)
