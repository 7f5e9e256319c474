// Internal launchers of the MoE kernels.  Each enqueues on stream `s` and returns the
// launch status; argument checking happens in the C ABI layer (moe_abi.cpp) before these
// are called.  dtype: 0 = fp32, 1 = bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Flat assignments handled by one dispatch tile: a multiple of k, at most kTileMax, so the
// k slots of a token never straddle two tiles.
constexpr int kTileMax = 512;
inline int64_t dispatch_tile_entries(int64_t k) { return (kTileMax / k) * k; }
inline int64_t dispatch_ntiles(int64_t T, int64_t k) {
  const int64_t te = dispatch_tile_entries(k);
  return (T * k + te - 1) / te;
}

hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t s);

// S1.  status_zero (nullable): an int32 the launch also sets to 0 before the logits are
// complete (the top-k status counter), without a launch of its own where it can.
hipError_t launch_router_logits(int dtype, const void* x, const void* w, const float* b,
                                float* logits, int64_t T, int64_t d, int64_t E,
                                int32_t* status_zero, hipStream_t s);
// S2
// sel_bias (nullable): selection-only bias.  n_groups > 1: group-limited selection keeping
// topk_groups groups (n_groups <= min(E, 64), dividing E).
hipError_t launch_topk(const float* logits, const float* sel_bias, int64_t T, int64_t E,
                       int64_t k, int n_groups, int topk_groups, int32_t* idx, float* w,
                       int32_t* status, hipStream_t s);

// S3-S5.  C is the effective capacity (1 <= C <= T when T > 0); R the row bound.
struct DispatchArgs {
  const int32_t* topk_idx;
  const void* x;
  int64_t T, d, E, k, C, R;
  int elt_bytes;
  bool slot_major;     // visit assignments slot-major instead of token-major
  bool pad;            // C slots per expert (offsets e * C, empty slots zero rows)
  int32_t* tile_hist;  // [ntiles, E]
  int32_t* tile_base;  // [ntiles, E]
  int32_t* routed;     // [E]
  int32_t* kept;       // [E]
  int32_t* offsets;    // [E+1]
  int32_t* src_token;  // [R]
  int32_t* src_slot;   // [R], nullable: slot of the assignment each kept row holds
  int32_t* dest_row;   // [T*k]
  int32_t* drops;      // [k+2]
  void* x_perm;        // [R, d]; null: tables only, no row copies
  // nullable: also write the grouped GEMMs' tile table of row height table_bm (at most
  // table_m_max entries, launch_expert_ffn's layout) from the offsets
  int32_t* table = nullptr;
  int table_bm = 0;
  int64_t table_m_max = 0;
};
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);
// The dispatch of T * k assignments over E experts runs in one block (no per-tile scratch
// tables) when it holds at most 2048 assignments over at most 256 experts.  (Measured per
// call: 5 us for 128 assignments, 9 us for 2048, against about 14 us for the three tiled
// kernels; 17 and 21 us for 4096 and 8192, where the tiled kernels are faster.)
constexpr int64_t kFusedDispatchEntries = 2048;
constexpr int64_t kFusedDispatchMaxE = 256;
inline bool dispatch_fused(int64_t T, int64_t k, int64_t E) {
  return T * k > 0 && T * k <= kFusedDispatchEntries && E <= kFusedDispatchMaxE;
}
// The static scratch of moe_dispatch_no_workspace on the current device: its address
// (looked up once per device) and size in bytes.
hipError_t dispatch_scratch(void** ptr, size_t* bytes);

// S6-S7.  The grouped GEMMs run over a device-side tile table (expert, first row) of
// row-tile height bm with at most m_max entries.
struct FfnPlan {
  bool small;      // decode-sized experts (weight streaming)
  int tile;        // 0 decode, 1 prefill 256 rows, 2 prefill 320 rows
  int bm;
  int64_t m_max;   // upper bound on m-tiles over all experts
  int down_split;  // 1, or the most pieces a tail tile of the down GEMM splits into
  int64_t down_pieces_max;  // bound on those pieces (slots of partial sums)
  bool stream_b;   // weight loads carry the non-temporal hint (each line read by ~1 tile)
  int group_cap;   // n-tiles per launch-order group (each XCD walks groups of m x group)
};
// pad: every expert holds exactly C rows (offsets e * C).  d, F and the element size
// decide whether the down GEMM splits its reduction.
FfnPlan ffn_plan(int64_t T, int64_t E, int64_t k, int64_t C, int64_t R, bool pad, int64_t d,
                 int64_t F, int64_t elt);
inline int64_t ffn_table_ints(const FfnPlan& p) { return 1 + 2 * p.m_max; }
// Upper bound on the blocks of one grouped-GEMM launch of plan p (512 threads each).
int64_t ffn_max_blocks(const FfnPlan& p, int64_t d, int64_t F);
// CUs the tail split of the down GEMM fills (MI355X: 256).
constexpr int kSplitCUs = 256;
// fp32 partial sums of the down GEMM's split tail tiles: down_pieces_max slots of
// bm x 256 floats (0 bytes when it does not split)
inline int64_t ffn_down_acc_bytes(const FfnPlan& p) {
  return p.down_split > 1 ? p.down_pieces_max * p.bm * 256 * 4 : 0;
}

struct FfnArgs {
  int dtype;
  const void* x_perm;
  const void* x;            // with src_rows: the gate/up GEMM reads x[src_rows[r]] for row r
  const int32_t* src_rows;  // nullable; [R] token of each row (-1: empty padded slot)
  const int32_t* offsets;  // [E+1]
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  int64_t T, d, E, k, F, C, R;
  bool pad;
  void* h;               // [R, F]
  int32_t* sched;        // ffn_table_ints() ints
  void* y_perm;          // [R, d]
  float* down_acc;       // ffn_down_acc_bytes() of fp32 partial sums (tail split)
  bool table_ready;      // sched already holds this call's tile table (skip rebuilding it)
};
// S1 through the grouped-GEMM pipeline in dense mode (64 x 128 tiles, fp32 out + bias),
// for shapes with enough tiles (router_gemm_suits).
bool router_gemm_suits(int64_t T, int64_t E);
hipError_t launch_router_gemm(int dtype, const void* x, const void* w, const float* b,
                              float* logits, int64_t T, int64_t d, int64_t E, hipStream_t s);

// which: 1 = gate/up GEMM (x_perm -> h), 2 = down GEMM (h -> y_perm), 3 = both.  Each
// call first rebuilds the tile table from `offsets`, unless a.table_ready says an earlier
// call on the same stream built it from the same offsets.
hipError_t launch_expert_ffn(const FfnArgs& a, int which, hipStream_t s);

// S8
hipError_t launch_combine(int dtype, const void* y_perm, const int32_t* dest_row,
                          const float* topk_w, void* out, int64_t T, int64_t d, int64_t k,
                          hipStream_t s);

// Observability: routed_by_slot / kept_by_slot [k, E] (zeroed here first).
hipError_t launch_slot_counts(const int32_t* idx, const int32_t* dest_row, int64_t T,
                              int64_t k, int64_t E, int32_t* routed_by_slot,
                              int32_t* kept_by_slot, hipStream_t s);

}  // namespace moe
