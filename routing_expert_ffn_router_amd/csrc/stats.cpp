// Host-side records of one layer's routing: the per-layer expert statistics, the per-slot
// record and the load of a placement of the experts over ranks and nodes.  Plain C++ over
// host arrays that the caller copied back from the device; nothing here touches the GPU.
// (The memory record by phase, moe_workspace_phases, sits with the workspace layout in
// moe_abi.cpp.)
//
// [EP-checks] airouter.kz, "Expert parallelism in MoE needs measurements before launch":
//   "Mean expert load proves almost nothing" -- the per-layer record (counts per expert,
//     p50, p95, max, max over mean, the share of the busiest 5 % of the experts, drops);
//   "Top-2 does not insure against hot experts" -- look at each choice separately, and at
//     which choices get dropped;
//   "Expert and GPU can be balanced differently" -- load per rank and per node under a
//     placement of the experts.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "../../include/moe.h"

namespace {

bool counts_ok(int64_t n, const int32_t* v) {
  for (int64_t i = 0; i < n; ++i)
    if (v[i] < 0) return false;
  return true;
}

}  // namespace

extern "C" {

int moe_expert_stats(int64_t T, int64_t k, int64_t E, const int32_t* routed_counts,
                     const int32_t* tokens_per_expert, moe_expert_stats_t* out) {
  if (T < 0 || k < 1 || E < 1 || !routed_counts || !out) return MOE_ERR_INVALID_ARG;
  if (!counts_ok(E, routed_counts)) return MOE_ERR_INVALID_ARG;
  if (tokens_per_expert) {
    if (!counts_ok(E, tokens_per_expert)) return MOE_ERR_INVALID_ARG;
    for (int64_t e = 0; e < E; ++e)
      if (tokens_per_expert[e] > routed_counts[e]) return MOE_ERR_INVALID_ARG;
  }
  std::vector<int64_t> s(routed_counts, routed_counts + E);
  std::sort(s.begin(), s.end());
  int64_t total = 0;
  for (int64_t v : s) total += v;
  // nearest rank: the ceil(q E)-th smallest count (q E in IEEE double, as ceil() sees it)
  auto nearest_rank = [&](double q) {
    int64_t r = (int64_t)ceil(q * (double)E) - 1;
    return s[(size_t)std::max<int64_t>(0, r)];
  };
  out->active_tokens = T;
  out->top_k = k;
  out->experts = E;
  out->routed = total;
  out->expert_p50 = nearest_rank(0.50);
  out->expert_p95 = nearest_rank(0.95);
  out->expert_max = s.back();
  out->expert_mean = (double)total / (double)E;
  out->expert_max_to_mean = total > 0 ? (double)s.back() / out->expert_mean : NAN;
  // the busiest ceil(5 % of E) experts and their share of the routed assignments
  const int64_t top = (int64_t)ceil(0.05 * (double)E);
  int64_t top_sum = 0;
  for (int64_t i = 0; i < top; ++i) top_sum += s[(size_t)(E - 1 - i)];
  out->top_5_percent_experts = top;
  out->top_5_percent_expert_share = total > 0 ? (double)top_sum / (double)total : 0.0;
  int64_t kept = 0, active = 0, dropped = 0;
  for (int64_t e = 0; e < E; ++e) {
    const int64_t c = tokens_per_expert ? tokens_per_expert[e] : routed_counts[e];
    kept += c;
    active += c > 0;
    dropped += routed_counts[e] - c;
  }
  out->kept_rows = kept;
  out->active_experts = active;
  out->dropped_tokens = dropped;
  return MOE_OK;
}

int moe_slot_stats(int64_t T, int64_t k, int64_t E, const int32_t* routed_by_slot,
                   const int32_t* kept_by_slot, double* slot_max_to_mean,
                   double* drop_share_per_slot) {
  if (T < 0 || k < 1 || E < 1 || !routed_by_slot || !kept_by_slot || !slot_max_to_mean ||
      !drop_share_per_slot)
    return MOE_ERR_INVALID_ARG;
  if (!counts_ok(k * E, routed_by_slot) || !counts_ok(k * E, kept_by_slot))
    return MOE_ERR_INVALID_ARG;
  std::vector<int64_t> dropped(k, 0);
  int64_t dropped_all = 0;
  for (int64_t j = 0; j < k; ++j) {
    int64_t mx = 0;
    for (int64_t e = 0; e < E; ++e) {
      const int64_t r = routed_by_slot[j * E + e], c = kept_by_slot[j * E + e];
      if (c > r) return MOE_ERR_INVALID_ARG;
      mx = std::max(mx, r);
      dropped[j] += r - c;
    }
    dropped_all += dropped[j];
    // each slot holds one choice of each of the T tokens: its mean per expert is T / E
    slot_max_to_mean[j] = T > 0 ? (double)mx / ((double)T / (double)E) : 0.0;
  }
  for (int64_t j = 0; j < k; ++j)
    drop_share_per_slot[j] = dropped_all > 0 ? (double)dropped[j] / (double)dropped_all : 0.0;
  return MOE_OK;
}

int moe_placement_load(int64_t E, const int32_t* routed_counts, const int32_t* placement,
                       int64_t n_ranks, int64_t ranks_per_node, int64_t* rank_load,
                       int64_t* node_load, double* max_to_mean) {
  if (E < 1 || n_ranks < 1 || ranks_per_node < 0 || !routed_counts || !placement ||
      !rank_load || !max_to_mean)
    return MOE_ERR_INVALID_ARG;
  if (ranks_per_node > 0 && !node_load) return MOE_ERR_INVALID_ARG;
  if (!counts_ok(E, routed_counts)) return MOE_ERR_INVALID_ARG;
  for (int64_t e = 0; e < E; ++e)
    if (placement[e] < 0 || placement[e] >= n_ranks) return MOE_ERR_INVALID_ARG;
  int64_t total = 0;
  for (int64_t r = 0; r < n_ranks; ++r) rank_load[r] = 0;
  for (int64_t e = 0; e < E; ++e) {
    rank_load[placement[e]] += routed_counts[e];
    total += routed_counts[e];
  }
  auto ratio = [&](const int64_t* v, int64_t n) {
    if (total == 0) return 0.0;
    int64_t mx = 0;
    for (int64_t i = 0; i < n; ++i) mx = std::max(mx, v[i]);
    return (double)mx / ((double)total / (double)n);
  };
  max_to_mean[0] = ratio(rank_load, n_ranks);
  max_to_mean[1] = 0.0;
  if (ranks_per_node > 0) {
    const int64_t nodes = (n_ranks + ranks_per_node - 1) / ranks_per_node;
    for (int64_t n = 0; n < nodes; ++n) node_load[n] = 0;
    for (int64_t r = 0; r < n_ranks; ++r) node_load[r / ranks_per_node] += rank_load[r];
    max_to_mean[1] = ratio(node_load, nodes);
  }
  return MOE_OK;
}

}  // extern "C"
