/*
 * moe.h -- C ABI of one GPU's share of a Mixture-of-Experts layer on MI355X (gfx950).
 *
 * The layer: a router (logits GEMM, softmax top-k, renormalised gates), dispatch into
 * expert-contiguous buffers with capacity truncation, a grouped SwiGLU expert FFN, and a
 * gate-weighted combine back to token order.  Every call below only enqueues HIP kernels on
 * the given stream and returns; none synchronises, allocates or frees.
 *
 * Pages cited:
 *   [EP-serving] aiunderstanding.org, "Expert parallelism for MoE serving" (ru / wo / id).
 *   [EP-checks]  airouter.kz blog, "Expert parallelism in MoE needs measurements before
 *                launch" ("Экспертный параллелизм MoE требует замеров до запуска").
 *
 * Conventions shared by every entry point
 *   - Shapes: T tokens, d model width, E experts, k experts per token, F expert FFN width,
 *     capacity C (see moe_shape.capacity).
 *   - Layouts: row-major.  Weights use the nn.Linear convention [out_features, in_features]
 *     stacked over experts: w_router [E, d], w_gate and w_up [E, F, d], w_down [E, d, F],
 *     so every GEMM operand is contiguous along its reduction axis.
 *   - Types: MOE_BF16 means bf16 activations and weights, fp32 logits, gates and
 *     accumulation, bf16 hidden/expert/layer outputs.  MOE_F32 means fp32 throughout.
 *     Index tables are int32.
 *   - Pointers are device pointers on the current HIP device unless marked "host".  Tensor
 *     pointers (x, weights, x_perm, y_perm, out) must be 16-byte aligned.
 *   - The caller owns every buffer; the library keeps no state between calls, so calls
 *     with distinct workspaces and outputs may run concurrently on different streams.
 *   - Errors: arguments are validated before anything is enqueued and a negative
 *     moe_status is returned on failure (nothing is launched).  A failed launch returns
 *     MOE_ERR_HIP.  T = 0 is valid.
 *   - Limits: 1 <= E <= 1024, 1 <= k <= min(E, 64), d and F multiples of 128 and at most
 *     2^20, T * k < 2^31, and a grouped-GEMM grid (rows and columns of the shape's tiles)
 *     within 2^32 threads; moe_workspace_size() returns 0 for a shape outside them.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad shape value, k > E, ... */
  MOE_ERR_UNSUPPORTED = -2, /* outside the limits above or unknown dtype */
  MOE_ERR_ALIGNMENT = -3,   /* a tensor pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = -4,   /* workspace null or smaller than moe_workspace_size() */
  MOE_ERR_HIP = -5,         /* a kernel launch failed */
  MOE_ERR_SCRATCH = -6      /* the shape needs more than the static dispatch scratch */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Variants of routing and dispatch, or-ed into moe_shape.flags; 0 selects the defaults
 * described at each entry point.
 *   MOE_FLAG_PAD_TO_CAPACITY  every expert owns C row slots: the kept rows of expert e are
 *       rows e*C + pos of x_perm / y_perm (expert_offsets[e] = e*C) and the slots past its
 *       kept count are zero rows, so the expert GEMMs run on E*C uniform rows.  Pages:
 *       [EP-serving] "Technical details" (fixed expert buffers keep the GEMM shapes
 *       regular) and [EP-checks] "Capacity factor changes quality, memory and tail
 *       latency" (padding spends memory and compute on empty slots).  Needs E*C < 2^31.
 *   MOE_FLAG_SLOT_MAJOR  drop priority visits assignments slot-major, (j, t): every first
 *       choice before any second choice, each slot in token order; kept rows of an expert
 *       are stored in that order.  [EP-checks] "Capacity factor changes quality, memory
 *       and tail latency" (which choices are dropped matters).
 *   MOE_FLAG_BIAS_SELECTION_ONLY  b_router shifts the selection only: logits = x w^T
 *       (no bias), the top-k uses the fp32 sums logits + b_router, and the gates use the
 *       unbiased logits of the selected experts.  [EP-checks] "Routing is a system-level
 *       decision" (balancing the load is part of routing). */
enum {
  MOE_FLAG_PAD_TO_CAPACITY = 1,
  MOE_FLAG_SLOT_MAJOR = 2,
  MOE_FLAG_BIAS_SELECTION_ONLY = 4
};

typedef struct {
  int64_t T;        /* tokens (rows of x) */
  int64_t d;        /* model width */
  int64_t E;        /* experts */
  int64_t k;        /* experts per token */
  int64_t F;        /* expert FFN width */
  int64_t capacity; /* per-expert capacity C; <= 0 means no limit (C = T) */
  int32_t dtype;    /* moe_dtype */
  int32_t flags;    /* MOE_FLAG_* bits; unknown bits are rejected */
  /* Group-limited top-k ([EP-checks] "Routing is a system-level decision": limiting how
   * many nodes a token reaches shapes the exchange).  With n_groups > 1 the experts form
   * n_groups groups of E / n_groups consecutive indices; a group's score is its best
   * selection logit; each token keeps its topk_groups best groups (ties to the lower
   * group) and picks its k experts among theirs.  n_groups 0 or 1: no limit (topk_groups
   * must then be 0).  Limits: n_groups <= 64 and divides E, 1 <= topk_groups <=
   * n_groups, k <= topk_groups * E / n_groups. */
  int32_t n_groups;
  int32_t topk_groups;
} moe_shape;

/* Drop counters written by moe_dispatch / moe_layer: drops[0] = dropped assignments,
 * drops[1 + j] = dropped assignments of slot j (j < k), drops[1 + k] = tokens whose k
 * assignments were all dropped.  Length k + 2. */

/* Regions of the workspace, for callers that want to read intermediate tables of
 * moe_layer (see moe_workspace_layout). */
typedef enum {
  MOE_WS_LOGITS = 0,  /* float [T, E] */
  MOE_WS_TOPK_IDX,    /* int32 [T, k] */
  MOE_WS_TOPK_W,      /* float [T, k] */
  MOE_WS_ROUTED,      /* int32 [E]   routed counts n_e */
  MOE_WS_KEPT,        /* int32 [E]   kept counts c_e */
  MOE_WS_OFFSETS,     /* int32 [E+1] */
  MOE_WS_SRC_TOKEN,   /* int32 [R]   R = moe_max_rows() */
  MOE_WS_DEST_ROW,    /* int32 [T, k] */
  MOE_WS_DROPS,       /* int32 [k+2] */
  MOE_WS_STATUS,      /* int32 [1] */
  MOE_WS_TILE_HIST,   /* internal */
  MOE_WS_TILE_BASE,   /* internal */
  MOE_WS_SCHED,       /* internal */
  MOE_WS_X_PERM,      /* [R, d] */
  MOE_WS_H,           /* [R, F] */
  MOE_WS_Y_PERM,      /* [R, d] */
  MOE_WS_DOWN_ACC,    /* internal: fp32 partial sums of the down GEMM's split tail tiles */
  MOE_WS_COUNT
} moe_ws_region;

/* Per-expert capacity from a capacity factor ([EP-checks], "Capacity factor changes
 * quality, memory and tail latency": mean tokens per expert times the factor; the mean is
 * T*k/E by the section "Mean expert load proves almost nothing").  Returns
 * ceil(((cf * T) * k) / E) evaluated in IEEE double; 0 (no limit) when cf <= 0; -1 when T < 0,
 * k < 1 or E < 1, cf is not finite or the result does not fit int64.  Host function. */
int64_t moe_capacity(int64_t T, int64_t k, int64_t E, double cf);

/* Row slots R of x_perm, y_perm and src_token: min(T*k, E*C) with C = T when unlimited,
 * or E*C with MOE_FLAG_PAD_TO_CAPACITY ([EP-serving] "Technical details": expert buffers
 * sized by the capacity; [EP-checks] "Capacity factor changes quality, memory and tail
 * latency": the capacity bounds what each expert's buffer must hold).  Returns -1 for an
 * invalid shape.  Host function. */
int64_t moe_max_rows(const moe_shape* shape);

/* Bytes of device workspace that any call below needs for this shape (the same size
 * serves all of them); 0 for an invalid shape.  [EP-checks] "Memory must be counted by
 * phase": the dispatch and combine buffers and the MoE temporaries are a line of their own
 * in the memory sheet, sized from the shape and capacity, not from the active parameters.
 * Host function. */
size_t moe_workspace_size(const moe_shape* shape);

/* Byte offsets (host array of MOE_WS_COUNT) of each region in the workspace; a region of
 * size 0 still gets an offset.  Regions are 256-byte aligned and laid out in the order of
 * moe_ws_region, so a region's size is bounded by the next offset (the last one by
 * moe_workspace_size).  [EP-checks] "Memory must be counted by phase" (which buffer each
 * stage holds).  Returns a moe_status.  Host function. */
int moe_workspace_layout(const moe_shape* shape, int64_t* offsets);

/* Human-readable name of a moe_status value (static string).  Host function. */
const char* moe_status_string(int status);

/* Phases of moe_layer at which [EP-checks] "Memory must be counted by phase" asks for the
 * memory held: before the MoE layer, after packing, after dispatch, after the expert
 * compute.  At expert-parallel size 1 the dispatch exchange moves nothing, so the figures
 * after packing and after dispatch are equal (a multi-GPU exchange would add its receive
 * buffers at the second). */
typedef enum {
  MOE_PHASE_BEFORE_LAYER = 0,
  MOE_PHASE_AFTER_PACK,     /* router tables, dispatch tables, x_perm when it is copied */
  MOE_PHASE_AFTER_DISPATCH, /* equal to MOE_PHASE_AFTER_PACK on one GPU */
  MOE_PHASE_AFTER_EXPERTS,  /* + the tile table, h, y_perm and any split-reduction slots */
  MOE_PHASE_COUNT
} moe_phase;

/* Bytes of the workspace that moe_layer has written by the end of each moe_phase
 * ([EP-checks] "Memory must be counted by phase"), as sums of the exact sizes of the
 * regions each stage writes (moe_ws_region; row regions at their bound R = moe_max_rows,
 * so these are upper bounds of what one call touches), assuming the optional outputs of
 * moe_layer (routed_counts, tokens_per_expert, drops, status) are NULL and so kept in the
 * workspace.  A gathered layer (see moe_layer) does not count x_perm.  The workspace itself
 * is allocated once by the caller: these figures say how much of it each phase needs.
 *   bytes  host array of MOE_PHASE_COUNT int64, out.
 * Returns a moe_status.  Host function. */
int moe_workspace_phases(const moe_shape* shape, int64_t* bytes);

/* S9: the per-layer expert statistics record of [EP-checks] "Mean expert load proves
 * almost nothing" (counts per expert after top-k, mean = sum / E, p50, p95, max, max over
 * mean, the share held by the busiest 5 % of the experts, drops).  Readings: the record is
 * over routed counts n_e (before capacity truncation, so a hot expert shows above the
 * capacity); p50 and p95 are nearest ranks, the ceil(q E)-th smallest count with q E
 * evaluated in IEEE double; the busiest 5 % are the ceil(0.05 E) largest counts. */
typedef struct {
  int64_t active_tokens;             /* T */
  int64_t top_k;                     /* k */
  int64_t experts;                   /* E */
  int64_t routed;                    /* sum of n_e */
  int64_t expert_p50;                /* nearest-rank median of n_e */
  int64_t expert_p95;                /* nearest-rank 95th percentile of n_e */
  int64_t expert_max;                /* max n_e */
  double expert_mean;                /* sum n_e / E */
  double expert_max_to_mean;         /* max / mean; NaN when nothing was routed */
  int64_t top_5_percent_experts;     /* ceil(0.05 E) */
  double top_5_percent_expert_share; /* their share of sum n_e; 0 when nothing was routed */
  int64_t kept_rows;                 /* sum c_e (sum n_e without tokens_per_expert) */
  int64_t active_experts;            /* experts with c_e > 0 */
  int64_t dropped_tokens;            /* dropped assignments, sum (n_e - c_e) */
} moe_expert_stats_t;

/* Fill *out from host copies of the counts of one layer.
 *   routed_counts      [E] int32 host, n_e >= 0
 *   tokens_per_expert  [E] int32 host, nullable: c_e with 0 <= c_e <= n_e (NULL: no drops)
 * Returns MOE_ERR_INVALID_ARG for T < 0, k < 1, E < 1, null pointers or counts outside
 * those ranges.  Host function. */
int moe_expert_stats(int64_t T, int64_t k, int64_t E, const int32_t* routed_counts,
                     const int32_t* tokens_per_expert, moe_expert_stats_t* out);

/* Per-slot record ([EP-checks] "Top-2 does not insure against hot experts": the second
 * choice can pile onto the same hot experts, and which choices get dropped matters), from
 * host copies of moe_slot_counts' tables.
 *   routed_by_slot, kept_by_slot  [k, E] int32 host (kept <= routed entry by entry)
 *   slot_max_to_mean    [k] double out: max_e routed_by_slot[j][e] / (T / E), the
 *                       imbalance of the (j+1)-th choice alone (0 when T = 0)
 *   drop_share_per_slot [k] double out: dropped assignments of slot j over all dropped
 *                       ones (0 when nothing was dropped)
 * Returns a moe_status.  Host function. */
int moe_slot_stats(int64_t T, int64_t k, int64_t E, const int32_t* routed_by_slot,
                   const int32_t* kept_by_slot, double* slot_max_to_mean,
                   double* drop_share_per_slot);

/* Load per rank and per node under a placement of the experts ([EP-checks] "Expert and GPU
 * can be balanced differently": balanced experts do not make balanced GPUs).
 *   routed_counts  [E] int32 host
 *   placement      [E] int32 host: rank holding expert e, in [0, n_ranks)
 *   ranks_per_node 0: no node figures; else ranks r * ranks_per_node ... form node r
 *   rank_load      [n_ranks] int64 out: sum of n_e over the rank's experts
 *   node_load      [ceil(n_ranks / ranks_per_node)] int64 out (nullable when
 *                  ranks_per_node is 0)
 *   max_to_mean    [2] double out: max over mean of the rank loads, then of the node loads
 *                  (0 when nothing was routed or without nodes)
 * Returns a moe_status.  Host function. */
int moe_placement_load(int64_t E, const int32_t* routed_counts, const int32_t* placement,
                       int64_t n_ranks, int64_t ranks_per_node, int64_t* rank_load,
                       int64_t* node_load, double* max_to_mean);

/*
 * moe_route -- S1 router logits and S2 top-k gating.
 * [EP-serving] "Deep dive": a router picks the top-k experts (often 1 or 2) of each token.
 * Layer specification: logits L = x w_router^T + b_router (fp32); the k largest logits
 * per token under (value descending, expert index ascending), -0.0 equal to +0.0; gates
 * w_j = exp(L_j - L_max) / sum over the k selected exp(L_i - L_max) (softmax restricted to
 * the selection and renormalised).  With MOE_FLAG_BIAS_SELECTION_ONLY the bias enters the
 * selection only; with n_groups > 1 the selection is group-limited (see moe_shape).
 *   x          [T, d] dtype          (unused when logits_given)
 *   w_router   [E, d] dtype          (unused when logits_given)
 *   b_router   [E] float, nullable
 *   logits     [T, E] float: output, or input when logits_given != 0
 *   topk_idx   [T, k] int32 out, slot 0 = best expert
 *   topk_w     [T, k] float out
 *   status     [1] int32 out, nullable: number of tokens with a non-finite logit (their
 *              selection and gates are then unspecified)
 */
int moe_route(const moe_shape* shape, const void* x, const void* w_router,
              const float* b_router, float* logits, int logits_given, int32_t* topk_idx,
              float* topk_w, int32_t* status, hipStream_t stream);

/*
 * moe_dispatch -- S3-S5: the single-GPU stand-in of the dispatch all-to-all.
 * [EP-serving] "Technical details" (tokens go to the experts they chose; experts have
 * capacity-limited buffers; overflow is dropped) and [EP-checks] "Capacity factor changes
 * quality, memory and tail latency" (overflow is dropped before the exchange).
 * Drop priority: first come, first kept in token order.  The assignment (t, j) -> e is
 * kept iff fewer than C earlier assignments (token-major order, or slot-major with
 * MOE_FLAG_SLOT_MAJOR) went to e.  Kept rows of expert e fill rows [expert_offsets[e],
 * expert_offsets[e] + tokens_per_expert[e]) of x_perm in that order; expert_offsets is
 * the exclusive scan of tokens_per_expert, or e*C with MOE_FLAG_PAD_TO_CAPACITY (then the
 * other slots of x_perm are zero rows).  Entries of topk_idx outside [0, E) are dropped.
 *   topk_idx          [T, k] int32 in
 *   x                 [T, d] dtype in
 *   workspace         moe_workspace_size() bytes; workspace_bytes its size
 *   routed_counts     [E] int32 out: n_e, assignments routed to e
 *   tokens_per_expert [E] int32 out: c_e = min(n_e, C)
 *   expert_offsets    [E+1] int32 out: exclusive scan of c_e
 *   src_token         [R] int32 out: token of each kept row, -1 for every other slot
 *   src_slot          [R] int32 out, nullable: slot j of the assignment (t, j) each kept
 *                     row holds, -1 for every other slot (dest_row inverted:
 *                     dest_row[src_token[r], src_slot[r]] = r)
 *   dest_row          [T, k] int32 out: row of each assignment in x_perm, -1 if dropped
 *   drops             [k+2] int32 out (see above)
 *   x_perm            [R, d] dtype out: x_perm[r] = x[src_token[r]] for kept rows; nullable:
 *                     NULL builds the tables only (no row is copied, x may then be NULL),
 *                     for moe_expert_gate_up_gathered
 */
int moe_dispatch(const moe_shape* shape, const int32_t* topk_idx, const void* x,
                 void* workspace, size_t workspace_bytes, int32_t* routed_counts,
                 int32_t* tokens_per_expert, int32_t* expert_offsets, int32_t* src_token,
                 int32_t* src_slot, int32_t* dest_row, int32_t* drops, void* x_perm,
                 hipStream_t stream);

/*
 * moe_dispatch_no_workspace -- moe_dispatch for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same operation, arguments and results as moe_dispatch, without the workspace.  The
 * dispatch's scratch tables (per-tile expert histogram and its per-expert scan, int32
 * [ntiles, E] each, 256-byte aligned, ntiles = ceil(T*k / (floor(512 / k) * k))) live in a
 * static array of MOE_DISPATCH_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends.  Calls on one GPU share that array: calls that overlap on one
 * GPU (concurrent streams, or threads) race and must not be made.  Shapes whose two tables
 * need more than the array holds return MOE_ERR_SCRATCH before anything is enqueued.  The
 * first call on a device looks up that device's copy of the array (no allocation); a
 * failed lookup returns MOE_ERR_HIP.  Nothing here allocates or frees memory.
 */
#define MOE_DISPATCH_SCRATCH_BYTES (8u << 20)
int moe_dispatch_no_workspace(const moe_shape* shape, const int32_t* topk_idx, const void* x,
                              int32_t* routed_counts, int32_t* tokens_per_expert,
                              int32_t* expert_offsets, int32_t* src_token, int32_t* src_slot,
                              int32_t* dest_row, int32_t* drops, void* x_perm,
                              hipStream_t stream);

/*
 * moe_expert_ffn -- S6-S7: grouped SwiGLU FFN over the expert-contiguous rows.
 * [EP-serving] "Deep dive" (each expert is a small feed-forward network) and "Technical
 * details" (expert buffers keep the GEMM shapes regular); layer specification: for rows r
 * of expert e, h = silu(x_perm[r] w_gate[e]^T) * (x_perm[r] w_up[e]^T), rounded to dtype,
 * and y_perm[r] = h w_down[e]^T.  Row counts per expert are read on the device from
 * expert_offsets; rows >= expert_offsets[E] are not written.
 *   x_perm          [R, d] dtype in
 *   expert_offsets  [E+1] int32 in (non-decreasing, expert_offsets[E] <= R)
 *   w_gate, w_up    [E, F, d] dtype; w_down [E, d, F] dtype
 *   workspace       holds h [R, F] and the tile schedule
 *   y_perm          [R, d] dtype out
 */
int moe_expert_ffn(const moe_shape* shape, const void* x_perm, const int32_t* expert_offsets,
                   const void* w_gate, const void* w_up, const void* w_down, void* workspace,
                   size_t workspace_bytes, void* y_perm, hipStream_t stream);

/*
 * moe_expert_gate_up -- S6 alone: h = silu(x_perm w_gate[e]^T) * (x_perm w_up[e]^T) for
 * the rows of each expert, rounded to dtype (same sources as moe_expert_ffn).  One grouped
 * GEMM launch after a one-block tile-table launch.
 *   h  [R, F] dtype out (rows >= expert_offsets[E] not written)
 */
int moe_expert_gate_up(const moe_shape* shape, const void* x_perm,
                       const int32_t* expert_offsets, const void* w_gate, const void* w_up,
                       void* workspace, size_t workspace_bytes, void* h, hipStream_t stream);

/*
 * moe_expert_gate_up_gathered -- S6 reading the token rows straight from x: h[r] =
 * silu(x[src_token[r]] w_gate[e]^T) * (x[src_token[r]] w_up[e]^T) for the rows of each
 * expert (the pack step of [EP-checks] "All-to-all must be profiled separately from
 * compute" fused into the GEMM's loads, so x_perm is neither written nor read).
 *   x          [T, d] dtype in; src_token [R] int32 in (from moe_dispatch)
 *   h          [R, F] dtype out (rows >= expert_offsets[E], and empty padded slots, whose
 *              src_token is -1, are unspecified)
 * Needs T * d * sizeof(dtype) < 2^31 (MOE_ERR_UNSUPPORTED otherwise).
 */
int moe_expert_gate_up_gathered(const moe_shape* shape, const void* x,
                                const int32_t* src_token, const int32_t* expert_offsets,
                                const void* w_gate, const void* w_up, void* workspace,
                                size_t workspace_bytes, void* h, hipStream_t stream);

/*
 * moe_expert_down -- S7 alone: y_perm[r] = h[r] w_down[e]^T for the rows of each expert
 * (same sources as moe_expert_ffn).  One grouped GEMM launch after a one-block tile-table
 * launch.  For shapes whose down GEMM has few, long tiles (at most m-tiles x ceil(d / 256)
 * of them, fewer than two rounds of the 256 CUs), the tiles that fall into the last,
 * partial round (counted on the device) split their reduction axis into up to 8 pieces,
 * each storing its tile of fp32 partial sums into a slot of the workspace region
 * MOE_WS_DOWN_ACC; one more launch adds each tile's slots in piece order and converts the
 * sums to y_perm, so the result does not depend on which piece finished first.  Such shapes
 * get a non-empty MOE_WS_DOWN_ACC (at most 256 slots of BM x 256 floats, BM the row-tile
 * height) from moe_workspace_size.
 *   h      [R, F] dtype in
 *   y_perm [R, d] dtype out (rows >= expert_offsets[E] not written)
 */
int moe_expert_down(const moe_shape* shape, const void* h, const int32_t* expert_offsets,
                    const void* w_down, void* workspace, size_t workspace_bytes, void* y_perm,
                    hipStream_t stream);

/*
 * moe_combine -- S8: gate-weighted sum back to token order, without atomics.
 * [EP-serving] "Technical details" (the combine step returns expert outputs to their
 * tokens); layer specification: out[t] = sum over slots j = 0..k-1 in order, skipping
 * dropped ones (dest_row < 0), of topk_w[t, j] * y_perm[dest_row[t, j]], accumulated in
 * fp32.  Gates of dropped assignments are not renormalised; a token with every slot dropped
 * gets a zero row.
 *   y_perm [R, d] dtype in; dest_row [T, k] int32 in; topk_w [T, k] float in
 *   out    [T, d] dtype out
 */
int moe_combine(const moe_shape* shape, const void* y_perm, const int32_t* dest_row,
                const float* topk_w, void* out, hipStream_t stream);

/*
 * moe_slot_counts -- routing observability ([EP-checks] "Mean expert load proves almost
 * nothing": look past the mean, at the second choice and at what gets dropped).
 * routed_by_slot[j * E + e] = tokens whose slot j chose expert e; kept_by_slot likewise
 * for assignments with dest_row >= 0.  Entries of topk_idx outside [0, E) are not
 * counted.
 *   topk_idx [T, k] int32 in; dest_row [T, k] int32 in
 *   routed_by_slot, kept_by_slot [k, E] int32 out
 */
int moe_slot_counts(const moe_shape* shape, const int32_t* topk_idx, const int32_t* dest_row,
                    int32_t* routed_by_slot, int32_t* kept_by_slot, hipStream_t stream);

/*
 * moe_layer -- the whole layer: moe_route, moe_dispatch, the expert GEMMs and moe_combine on
 * one stream, with every intermediate in the workspace (regions in moe_ws_region).  This
 * is the expert-parallel-size-1 configuration of [EP-checks] "All-to-all must be profiled
 * separately from compute": every expert is local and no all-to-all runs.  With packed
 * rows (no MOE_FLAG_PAD_TO_CAPACITY) and T * d * sizeof(dtype) < 2^31 the gate/up GEMM
 * gathers the token rows itself (moe_expert_gate_up_gathered) and the x_perm region is
 * left unwritten.  The dispatch also writes the grouped GEMMs' tile table from the offsets
 * it computes, and both GEMMs read it from the workspace.
 *   out               [T, d] dtype out
 *   routed_counts, tokens_per_expert [E] int32 out, nullable (then kept in the workspace)
 *   drops             [k+2] int32 out, nullable
 *   status            [1] int32 out, nullable (non-finite logit count, as in moe_route)
 */
int moe_layer(const moe_shape* shape, const void* x, const void* w_router,
              const float* b_router, const void* w_gate, const void* w_up, const void* w_down,
              void* workspace, size_t workspace_bytes, void* out, int32_t* routed_counts,
              int32_t* tokens_per_expert, int32_t* drops, int32_t* status,
              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
