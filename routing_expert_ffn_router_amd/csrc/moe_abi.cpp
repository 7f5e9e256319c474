// C ABI of the MoE layer: argument validation, workspace layout and the call sequence of
// each entry point.  Every check happens before anything is enqueued; kernels only see
// arguments that passed them.  See include/moe.h for the contract of each function.
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

constexpr int64_t kAlign = 256;
constexpr int64_t kMaxE = 1024;
constexpr int64_t kMaxK = 64;

int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int elt_bytes(int32_t dtype) { return dtype == MOE_BF16 ? 2 : 4; }

int64_t eff_capacity(const moe_shape* s) {
  return (s->capacity <= 0 || s->capacity > s->T) ? s->T : s->capacity;
}

constexpr int32_t kKnownFlags =
    MOE_FLAG_PAD_TO_CAPACITY | MOE_FLAG_SLOT_MAJOR | MOE_FLAG_BIAS_SELECTION_ONLY;
constexpr int64_t kMaxGroups = 64;

bool padded(const moe_shape* s) { return (s->flags & MOE_FLAG_PAD_TO_CAPACITY) != 0; }
bool grouped(const moe_shape* s) { return s->n_groups > 1 && s->topk_groups < s->n_groups; }

int64_t max_rows(const moe_shape* s) {
  const int64_t a = s->T * s->k, b = s->E * eff_capacity(s);
  if (padded(s)) return b;
  return a < b ? a : b;
}

int check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->T < 0 || s->d <= 0 || s->E <= 0 || s->k <= 0 || s->F <= 0) return MOE_ERR_INVALID_ARG;
  if (s->flags & ~kKnownFlags) return MOE_ERR_INVALID_ARG;
  if (s->k > s->E) return MOE_ERR_INVALID_ARG;
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (s->E > kMaxE || s->k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (s->d % 128 != 0 || s->F % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (s->T > ((((int64_t)1 << 31) - 1) / s->k)) return MOE_ERR_UNSUPPORTED;  // T * k < 2^31
  if (s->d > ((int64_t)1 << 20) || s->F > ((int64_t)1 << 20)) return MOE_ERR_UNSUPPORTED;
  if (padded(s) && s->E * eff_capacity(s) >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  // group-limited selection
  if (s->n_groups < 0 || s->topk_groups < 0) return MOE_ERR_INVALID_ARG;
  if (s->n_groups <= 1) {
    if (s->topk_groups != 0) return MOE_ERR_INVALID_ARG;
  } else {
    if (s->n_groups > kMaxGroups || s->n_groups > s->E) return MOE_ERR_UNSUPPORTED;
    if (s->E % s->n_groups != 0) return MOE_ERR_INVALID_ARG;
    if (s->topk_groups < 1 || s->topk_groups > s->n_groups) return MOE_ERR_INVALID_ARG;
    if (s->k > (int64_t)s->topk_groups * (s->E / s->n_groups)) return MOE_ERR_INVALID_ARG;
  }
  // every grouped-GEMM launch within 2^32 threads (512 per block)
  const int64_t R = max_rows(s);
  const moe::FfnPlan plan = moe::ffn_plan(s->T, s->E, s->k, eff_capacity(s), R, padded(s),
                                          s->d, s->F, elt_bytes(s->dtype));
  if (moe::ffn_max_blocks(plan, s->d, s->F) >= ((int64_t)1 << 23)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

struct Layout {
  int64_t off[MOE_WS_COUNT];
  int64_t size[MOE_WS_COUNT];
  int64_t total;
};

Layout make_layout(const moe_shape* s) {
  Layout L;
  const int64_t T = s->T, E = s->E, k = s->k, R = max_rows(s), b = elt_bytes(s->dtype);
  const int64_t ntiles = moe::dispatch_ntiles(T, k);
  L.size[MOE_WS_LOGITS] = T * E * 4;
  L.size[MOE_WS_TOPK_IDX] = T * k * 4;
  L.size[MOE_WS_TOPK_W] = T * k * 4;
  L.size[MOE_WS_ROUTED] = E * 4;
  L.size[MOE_WS_KEPT] = E * 4;
  L.size[MOE_WS_OFFSETS] = (E + 1) * 4;
  L.size[MOE_WS_SRC_TOKEN] = R * 4;
  L.size[MOE_WS_DEST_ROW] = T * k * 4;
  L.size[MOE_WS_DROPS] = (k + 2) * 4;
  L.size[MOE_WS_STATUS] = 4;
  L.size[MOE_WS_TILE_HIST] = ntiles * E * 4;
  L.size[MOE_WS_TILE_BASE] = ntiles * E * 4;
  const moe::FfnPlan plan =
      moe::ffn_plan(T, E, k, eff_capacity(s), R, padded(s), s->d, s->F, b);
  L.size[MOE_WS_SCHED] = moe::ffn_table_ints(plan) * 4;
  L.size[MOE_WS_X_PERM] = R * s->d * b;
  L.size[MOE_WS_H] = R * s->F * b;
  L.size[MOE_WS_Y_PERM] = R * s->d * b;
  L.size[MOE_WS_DOWN_ACC] = moe::ffn_down_acc_bytes(plan);
  int64_t o = 0;
  for (int i = 0; i < MOE_WS_COUNT; ++i) {
    L.off[i] = o;
    o += align_up(L.size[i]);
  }
  L.total = o;
  return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

template <class P>
P* region(void* ws, const Layout& L, int r) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + L.off[r]);
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Rows of x addressed by 32-bit byte offsets in the gathered gate/up GEMM.
bool gather_fits(const moe_shape* s) {
  return s->T * s->d * elt_bytes(s->dtype) < ((int64_t)1 << 31);
}

// moe_layer lets the gate/up GEMM gather the token rows (x_perm is not written) with packed
// rows whose x fits 32-bit offsets.
bool layer_gathers(const moe_shape* s) { return !padded(s) && gather_fits(s); }

int check_workspace(const moe_shape* s, const void* ws, size_t bytes, Layout* L) {
  *L = make_layout(s);
  if (!ws || (int64_t)bytes < L->total) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

// Argument checks of the dispatch (everything but the scratch tables).
int check_dispatch_args(const moe_shape* s, const int32_t* topk_idx, const void* x,
                        const int32_t* routed_counts, const int32_t* tokens_per_expert,
                        const int32_t* expert_offsets, const int32_t* src_token,
                        const int32_t* dest_row, const int32_t* drops, const void* x_perm) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (!routed_counts || !tokens_per_expert || !expert_offsets || !drops)
    return MOE_ERR_INVALID_ARG;
  if (s->T > 0 && (!topk_idx || !src_token || !dest_row || (x_perm && !x)))
    return MOE_ERR_INVALID_ARG;
  if (s->T > 0 && x_perm && (!aligned16(x) || !aligned16(x_perm))) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

// The dispatch launches, with the scratch tables tile_hist / tile_base ([ntiles, E] int32
// each) from the workspace or from the static array.
// With table set, the dispatch also writes the grouped GEMMs' tile table of the layer's
// plan there (moe_layer).
int dispatch_launch(const moe_shape* s, const int32_t* topk_idx, const void* x,
                    int32_t* tile_hist, int32_t* tile_base, int32_t* routed_counts,
                    int32_t* tokens_per_expert, int32_t* expert_offsets, int32_t* src_token,
                    int32_t* src_slot, int32_t* dest_row, int32_t* drops, void* x_perm,
                    hipStream_t st, int32_t* table = nullptr) {
  moe::DispatchArgs a;
  a.topk_idx = topk_idx;
  a.x = x;
  a.T = s->T;
  a.d = s->d;
  a.E = s->E;
  a.k = s->k;
  a.C = eff_capacity(s);
  a.R = max_rows(s);
  a.elt_bytes = elt_bytes(s->dtype);
  a.slot_major = (s->flags & MOE_FLAG_SLOT_MAJOR) != 0;
  a.pad = padded(s);
  a.tile_hist = tile_hist;
  a.tile_base = tile_base;
  a.routed = routed_counts;
  a.kept = tokens_per_expert;
  a.offsets = expert_offsets;
  a.src_token = src_token;
  a.src_slot = src_slot;
  a.dest_row = dest_row;
  a.drops = drops;
  a.x_perm = x_perm;
  if (table) {
    const moe::FfnPlan plan = moe::ffn_plan(s->T, s->E, s->k, a.C, a.R, a.pad, s->d, s->F,
                                            a.elt_bytes);
    a.table = table;
    a.table_bm = plan.bm;
    a.table_m_max = plan.m_max;
  }
  return hip_status(moe::launch_dispatch(a, st));
}

int route_impl(const moe_shape* s, const void* x, const void* w_router, const float* b_router,
               float* logits, int logits_given, int32_t* idx, float* gates, int32_t* status,
               hipStream_t st) {
  hipError_t e;
  // the status counter starts at zero: cleared by the router launch when there is one
  if (logits_given || s->T == 0) {
    if (status && (e = moe::launch_zero_i32(status, 1, st)) != hipSuccess) return MOE_ERR_HIP;
    if (s->T == 0) return MOE_OK;
  }
  // with a selection-only bias the logits stay unbiased and the bias goes to the top-k
  const bool sel_only = (s->flags & MOE_FLAG_BIAS_SELECTION_ONLY) != 0;
  if (!logits_given) {
    e = moe::launch_router_logits(s->dtype, x, w_router, sel_only ? nullptr : b_router, logits,
                                  s->T, s->d, s->E, status, st);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  const int ng = grouped(s) ? s->n_groups : 1, mg = grouped(s) ? s->topk_groups : 1;
  return hip_status(moe::launch_topk(logits, sel_only ? b_router : nullptr, s->T, s->E, s->k,
                                     ng, mg, idx, gates, status, st));
}

}  // namespace

extern "C" {

int64_t moe_capacity(int64_t T, int64_t k, int64_t E, double cf) {
  if (T < 0 || k < 1 || E < 1 || !isfinite(cf)) return -1;
  if (!(cf > 0)) return 0;
  const double c = ceil(((cf * (double)T) * (double)k) / (double)E);
  if (!(c < 9.2233720368547758e18)) return -1;  // does not fit int64
  return (int64_t)c;
}

int64_t moe_max_rows(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return -1;
  return max_rows(s);
}

size_t moe_workspace_size(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return (size_t)make_layout(s).total;
}

int moe_workspace_layout(const moe_shape* s, int64_t* offsets) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (!offsets) return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(s);
  for (int i = 0; i < MOE_WS_COUNT; ++i) offsets[i] = L.off[i];
  return MOE_OK;
}

int moe_workspace_phases(const moe_shape* s, int64_t* bytes) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(s);
  // regions moe_layer writes in each stage (with its optional outputs kept in the workspace);
  // its dispatch also writes the grouped GEMMs' tile table, and the per-tile scratch tables
  // only where it runs tiled (not in one block)
  static const int kPack[] = {MOE_WS_LOGITS,    MOE_WS_TOPK_IDX, MOE_WS_TOPK_W,
                              MOE_WS_STATUS,    MOE_WS_ROUTED,   MOE_WS_KEPT,
                              MOE_WS_OFFSETS,   MOE_WS_SRC_TOKEN, MOE_WS_DEST_ROW,
                              MOE_WS_DROPS,     MOE_WS_SCHED};
  static const int kExperts[] = {MOE_WS_H, MOE_WS_Y_PERM, MOE_WS_DOWN_ACC};
  int64_t pack = 0;
  for (int r : kPack) pack += L.size[r];
  if (!moe::dispatch_fused(s->T, s->k, s->E))
    pack += L.size[MOE_WS_TILE_HIST] + L.size[MOE_WS_TILE_BASE];
  if (!layer_gathers(s)) pack += L.size[MOE_WS_X_PERM];  // the copy the gathering GEMM skips
  int64_t experts = pack;
  // an empty layer writes its counters and status only: the expert GEMMs do not launch
  if (s->T > 0)
    for (int r : kExperts) experts += L.size[r];
  bytes[MOE_PHASE_BEFORE_LAYER] = 0;
  bytes[MOE_PHASE_AFTER_PACK] = pack;
  bytes[MOE_PHASE_AFTER_DISPATCH] = pack;  // expert-parallel size 1: nothing is exchanged
  bytes[MOE_PHASE_AFTER_EXPERTS] = experts;
  return MOE_OK;
}

const char* moe_status_string(int st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_SCRATCH: return "shape needs more than the static dispatch scratch";
    default: return "unknown status";
  }
}

int moe_route(const moe_shape* s, const void* x, const void* w_router, const float* b_router,
              float* logits, int logits_given, int32_t* topk_idx, float* topk_w,
              int32_t* status, hipStream_t st) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (s->T > 0 && (!logits || !topk_idx || !topk_w)) return MOE_ERR_INVALID_ARG;
  if (!logits_given && s->T > 0) {
    if (!x || !w_router) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_ALIGNMENT;
  }
  return route_impl(s, x, w_router, b_router, logits, logits_given, topk_idx, topk_w, status,
                    st);
}

int moe_dispatch(const moe_shape* s, const int32_t* topk_idx, const void* x, void* ws,
                 size_t ws_bytes, int32_t* routed_counts, int32_t* tokens_per_expert,
                 int32_t* expert_offsets, int32_t* src_token, int32_t* src_slot,
                 int32_t* dest_row, int32_t* drops, void* x_perm, hipStream_t st) {
  int rc = check_dispatch_args(s, topk_idx, x, routed_counts, tokens_per_expert,
                               expert_offsets, src_token, dest_row, drops, x_perm);
  if (rc != MOE_OK) return rc;
  Layout L;
  if ((rc = check_workspace(s, ws, ws_bytes, &L)) != MOE_OK) return rc;
  return dispatch_launch(s, topk_idx, x, region<int32_t>(ws, L, MOE_WS_TILE_HIST),
                         region<int32_t>(ws, L, MOE_WS_TILE_BASE), routed_counts,
                         tokens_per_expert, expert_offsets, src_token, src_slot, dest_row,
                         drops, x_perm, st);
}

int moe_dispatch_no_workspace(const moe_shape* s, const int32_t* topk_idx, const void* x,
                              int32_t* routed_counts, int32_t* tokens_per_expert,
                              int32_t* expert_offsets, int32_t* src_token, int32_t* src_slot,
                              int32_t* dest_row, int32_t* drops, void* x_perm,
                              hipStream_t st) {
  int rc = check_dispatch_args(s, topk_idx, x, routed_counts, tokens_per_expert,
                               expert_offsets, src_token, dest_row, drops, x_perm);
  if (rc != MOE_OK) return rc;
  // the two scratch tables, each 256-byte aligned, in the static array
  const int64_t table = align_up(moe::dispatch_ntiles(s->T, s->k) * s->E * 4);
  if (2 * table > (int64_t)MOE_DISPATCH_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  void* scratch = nullptr;
  size_t bytes = 0;
  if (moe::dispatch_scratch(&scratch, &bytes) != hipSuccess) return MOE_ERR_HIP;
  if ((int64_t)bytes < 2 * table) return MOE_ERR_SCRATCH;
  int32_t* hist = static_cast<int32_t*>(scratch);
  int32_t* base = reinterpret_cast<int32_t*>(static_cast<char*>(scratch) + table);
  return dispatch_launch(s, topk_idx, x, hist, base, routed_counts, tokens_per_expert,
                         expert_offsets, src_token, src_slot, dest_row, drops, x_perm, st);
}

}  // extern "C"

namespace {

// Shared body of the expert-FFN entry points; which = 1 (gate/up), 2 (down), 3 (both).  The
// gate/up activations are x_perm, or, with src_rows, the rows src_rows[r] of x.
// With table_ready the workspace already holds the tile table of these offsets (moe_layer's
// dispatch wrote it).
int expert_ffn_impl(const moe_shape* s, int which, const void* x_perm, const void* x,
                    const int32_t* src_rows, void* h, const int32_t* expert_offsets,
                    const void* w_gate, const void* w_up, const void* w_down, void* ws,
                    size_t ws_bytes, void* y_perm, hipStream_t st, bool table_ready = false) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (s->T == 0) return MOE_OK;
  if (!expert_offsets) return MOE_ERR_INVALID_ARG;
  const void* act = src_rows ? x : x_perm;
  if ((which & 1) && (!act || !w_gate || !w_up || !h)) return MOE_ERR_INVALID_ARG;
  if ((which & 2) && (!w_down || !y_perm || !h)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(act) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(y_perm) || !aligned16(h))
    return MOE_ERR_ALIGNMENT;
  if (src_rows && !gather_fits(s)) return MOE_ERR_UNSUPPORTED;
  Layout L;
  if ((rc = check_workspace(s, ws, ws_bytes, &L)) != MOE_OK) return rc;
  moe::FfnArgs a;
  a.dtype = s->dtype;
  a.x_perm = x_perm;
  a.x = x;
  a.src_rows = src_rows;
  a.offsets = expert_offsets;
  a.w_gate = w_gate;
  a.w_up = w_up;
  a.w_down = w_down;
  a.T = s->T;
  a.d = s->d;
  a.E = s->E;
  a.k = s->k;
  a.F = s->F;
  a.C = eff_capacity(s);
  a.R = max_rows(s);
  a.pad = padded(s);
  a.h = h;
  a.sched = region<int32_t>(ws, L, MOE_WS_SCHED);
  a.y_perm = y_perm;
  a.down_acc = region<float>(ws, L, MOE_WS_DOWN_ACC);
  a.table_ready = table_ready;
  return hip_status(moe::launch_expert_ffn(a, which, st));
}

}  // namespace

extern "C" {

int moe_expert_ffn(const moe_shape* s, const void* x_perm, const int32_t* expert_offsets,
                   const void* w_gate, const void* w_up, const void* w_down, void* ws,
                   size_t ws_bytes, void* y_perm, hipStream_t st) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  Layout L;
  if (s->T > 0 && (rc = check_workspace(s, ws, ws_bytes, &L)) != MOE_OK) return rc;
  void* h = s->T > 0 ? region<void>(ws, L, MOE_WS_H) : nullptr;
  return expert_ffn_impl(s, 3, x_perm, nullptr, nullptr, h, expert_offsets, w_gate, w_up,
                         w_down, ws, ws_bytes, y_perm, st);
}

int moe_expert_gate_up(const moe_shape* s, const void* x_perm, const int32_t* expert_offsets,
                       const void* w_gate, const void* w_up, void* ws, size_t ws_bytes,
                       void* h, hipStream_t st) {
  return expert_ffn_impl(s, 1, x_perm, nullptr, nullptr, h, expert_offsets, w_gate, w_up,
                         nullptr, ws, ws_bytes, nullptr, st);
}

int moe_expert_gate_up_gathered(const moe_shape* s, const void* x, const int32_t* src_token,
                                const int32_t* expert_offsets, const void* w_gate,
                                const void* w_up, void* ws, size_t ws_bytes, void* h,
                                hipStream_t st) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (s->T > 0 && !src_token) return MOE_ERR_INVALID_ARG;
  return expert_ffn_impl(s, 1, nullptr, x, src_token, h, expert_offsets, w_gate, w_up,
                         nullptr, ws, ws_bytes, nullptr, st);
}

int moe_expert_down(const moe_shape* s, const void* h, const int32_t* expert_offsets,
                    const void* w_down, void* ws, size_t ws_bytes, void* y_perm,
                    hipStream_t st) {
  return expert_ffn_impl(s, 2, nullptr, nullptr, nullptr, const_cast<void*>(h), expert_offsets,
                         nullptr, nullptr, w_down, ws, ws_bytes, y_perm, st);
}

int moe_combine(const moe_shape* s, const void* y_perm, const int32_t* dest_row,
                const float* topk_w, void* out, hipStream_t st) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (s->T == 0) return MOE_OK;
  if (!y_perm || !dest_row || !topk_w || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y_perm) || !aligned16(out)) return MOE_ERR_ALIGNMENT;
  return hip_status(
      moe::launch_combine(s->dtype, y_perm, dest_row, topk_w, out, s->T, s->d, s->k, st));
}

int moe_slot_counts(const moe_shape* s, const int32_t* topk_idx, const int32_t* dest_row,
                    int32_t* routed_by_slot, int32_t* kept_by_slot, hipStream_t st) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (!routed_by_slot || !kept_by_slot) return MOE_ERR_INVALID_ARG;
  if (s->T > 0 && (!topk_idx || !dest_row)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_slot_counts(topk_idx, dest_row, s->T, s->k, s->E,
                                            routed_by_slot, kept_by_slot, st));
}

int moe_layer(const moe_shape* s, const void* x, const void* w_router, const float* b_router,
              const void* w_gate, const void* w_up, const void* w_down, void* ws,
              size_t ws_bytes, void* out, int32_t* routed_counts, int32_t* tokens_per_expert,
              int32_t* drops, int32_t* status, hipStream_t st) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (!w_router || !w_gate || !w_up || !w_down) return MOE_ERR_INVALID_ARG;
  if (s->T > 0 && (!x || !out)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(w_up) ||
      !aligned16(w_down) || !aligned16(out))
    return MOE_ERR_ALIGNMENT;
  Layout L;
  if ((rc = check_workspace(s, ws, ws_bytes, &L)) != MOE_OK) return rc;
  float* logits = region<float>(ws, L, MOE_WS_LOGITS);
  int32_t* idx = region<int32_t>(ws, L, MOE_WS_TOPK_IDX);
  float* gates = region<float>(ws, L, MOE_WS_TOPK_W);
  int32_t* routed = routed_counts ? routed_counts : region<int32_t>(ws, L, MOE_WS_ROUTED);
  int32_t* kept = tokens_per_expert ? tokens_per_expert : region<int32_t>(ws, L, MOE_WS_KEPT);
  int32_t* offsets = region<int32_t>(ws, L, MOE_WS_OFFSETS);
  int32_t* src = region<int32_t>(ws, L, MOE_WS_SRC_TOKEN);
  int32_t* dest = region<int32_t>(ws, L, MOE_WS_DEST_ROW);
  int32_t* dr = drops ? drops : region<int32_t>(ws, L, MOE_WS_DROPS);
  int32_t* stt = status ? status : region<int32_t>(ws, L, MOE_WS_STATUS);
  void* x_perm = region<void>(ws, L, MOE_WS_X_PERM);
  void* y_perm = region<void>(ws, L, MOE_WS_Y_PERM);

  rc = route_impl(s, x, w_router, b_router, logits, 0, idx, gates, stt, st);
  if (rc != MOE_OK) return rc;
  // packed rows: the gate/up GEMM gathers the token rows itself (x_perm is not written)
  const bool gathered = layer_gathers(s);
  void* x_copy = gathered ? nullptr : x_perm;
  rc = check_dispatch_args(s, idx, x, routed, kept, offsets, src, dest, dr, x_copy);
  if (rc != MOE_OK) return rc;
  // the dispatch also writes the grouped GEMMs' tile table from the offsets it computes
  rc = dispatch_launch(s, idx, x, region<int32_t>(ws, L, MOE_WS_TILE_HIST),
                       region<int32_t>(ws, L, MOE_WS_TILE_BASE), routed, kept, offsets, src,
                       nullptr, dest, dr, x_copy, st, region<int32_t>(ws, L, MOE_WS_SCHED));
  if (rc != MOE_OK) return rc;
  void* h = region<void>(ws, L, MOE_WS_H);
  rc = expert_ffn_impl(s, 1, gathered ? nullptr : x_perm, gathered ? x : nullptr,
                       gathered ? src : nullptr, h, offsets, w_gate, w_up, nullptr, ws,
                       ws_bytes, nullptr, st, /*table_ready=*/true);
  if (rc != MOE_OK) return rc;
  rc = expert_ffn_impl(s, 2, nullptr, nullptr, nullptr, h, offsets, nullptr, nullptr, w_down,
                       ws, ws_bytes, y_perm, st, /*table_ready=*/true);
  if (rc != MOE_OK) return rc;
  return moe_combine(s, y_perm, dest, gates, out, st);
}

}  // extern "C"
