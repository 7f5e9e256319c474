// S3-S5: the single-GPU stand-in of the dispatch all-to-all.
//
// [EP-serving] aiunderstanding.org, "Expert parallelism for MoE serving", section
// "Technical details": tokens go to the experts they chose, experts have capacity-limited
// buffers and overflow is dropped.  [EP-checks] airouter.kz, "Expert parallelism in MoE
// needs measurements before launch", section "Capacity factor changes quality, memory and
// tail latency": the overflow is dropped before the exchange, so every keep/drop decision
// below is final before a single row moves.
//
// Drop priority is first come, first kept: the assignments are visited in priority order
// -- token-major p = t * k + j by default, slot-major p = j * T + t (every first choice
// before any second choice) on request -- the visit list is stably counting-sorted by
// expert, and an assignment is kept iff its position among its expert's assignments is
// below the capacity C.
//
//   K3 tile_hist   per tile of the visit list, an LDS histogram over experts
//   K4 scan        per expert, the exclusive scan over tiles, then counts, capacity,
//                  offsets (exclusive scan over experts, or e * C when every expert owns C
//                  padded slots) and zeroed drop counters
//   K5 rank        per assignment, its position = tile base + earlier waves of the tile
//                  + rank inside the wave (wave ballots on the expert id bits); keep/drop,
//                  dest_row, src_token (and src_slot) and drop counters
//   K5c token_drop (slot-major only) tokens whose k assignments were all dropped
//   K5b gather     x_perm[r] = x[src_token[r]] with 16-byte vector copies; empty slots
//                  get src_token -1 (and, when padded, a zero row).  With packed rows and
//                  no copy requested, K5 marks the empty slots and K5b is not launched.
//   K345 fused     for at most 2048 assignments over at most 256 experts: K3-K5 (and the
//                  grouped GEMMs' tile table) in one block, one launch instead of three or
//                  four (the decode-sized and small prefill layers are launch-bound here).
// On request the scan (or the fused kernel) also writes the grouped GEMMs' tile table from
// the offsets it has just computed, which saves that table its own launch.
#include "common.h"
#include "kernels.h"

namespace moe {

// Index into topk_idx / dest_row [T, k] of visit position p.
__device__ inline int64_t visit_entry(int64_t p, int64_t T, int k, bool slot_major) {
  return slot_major ? (p % T) * k + p / T : p;
}

__global__ void __launch_bounds__(kTileMax)
tile_hist_kernel(const int32_t* __restrict__ idx, int64_t total, int64_t T, int te, int k,
                 int E, bool slot_major, int32_t* __restrict__ hist) {
  extern __shared__ int32_t s_cnt[];  // [E]
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_cnt[e] = 0;
  __syncthreads();
  const int64_t p = (int64_t)blockIdx.x * te + threadIdx.x;
  if ((int)threadIdx.x < te && p < total) {
    const int e = idx[visit_entry(p, T, k, slot_major)];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(int64_t)blockIdx.x * E + e] = s_cnt[e];
}

// Tile table of row-tile height bm for the grouped GEMMs (table[0] = tile count, capped at
// m_max; entry i = (expert, first row) at table[1 + 2i], table[2 + 2i]): expert e's rows
// are rows[e] from row0[e] on.  Every thread of the block calls it (it holds barriers); the
// threads with e < E bring their expert's values.
__device__ inline void write_tile_table(int e, int E, int row0, int rows, int bm, int m_max,
                                        int* smem, int32_t* __restrict__ table) {
  const int tiles = e < E ? rows / bm + (rows % bm != 0) : 0;
  int total;
  const int pre = block_exclusive_scan(tiles, smem, &total);
  if (threadIdx.x == 0) table[0] = total < m_max ? total : m_max;
  for (int i = 0; i < tiles && pre + i < m_max; ++i) {
    table[1 + 2 * (pre + i)] = e;
    table[2 + 2 * (pre + i)] = row0 + i * bm;
  }
}

// One block of 1024 threads.  Thread tid = part * E + e scans part `part` of expert e's
// tile counts (q parts per expert, q the smallest power of two >= the tile count, at most
// the largest with q * E <= 1024), so the
// per-expert scans over many tiles run q-wide; partial sums meet in LDS.  The threads with
// part 0 (tid = e) then hold the kept counts in expert order for the offsets scan.  With
// `table` set the block also writes the grouped GEMMs' tile table (write_tile_table).
__global__ void __launch_bounds__(1024)
scan_kernel(const int32_t* __restrict__ hist, int ntiles, int E, int C, int k, bool pad,
            int32_t* __restrict__ tile_base, int32_t* __restrict__ routed,
            int32_t* __restrict__ kept, int32_t* __restrict__ offsets,
            int32_t* __restrict__ drops, int32_t* __restrict__ table, int bm, int m_max) {
  __shared__ int smem[17];
  __shared__ int s_part[1024];
  int q = 1;
  while (q * 2 * E <= 1024 && q < ntiles) q *= 2;
  const int tid = threadIdx.x, part = tid / E, e = tid - part * E;
  const bool live = part < q;
  const int chunk = (ntiles + q - 1) / q;
  const int t_begin = part * chunk, t_end = min(ntiles, t_begin + chunk);
  int sum = 0;
  // unrolled so that several of the loads are in flight at once (the trip count is a
  // runtime value; rolled, each load waited for the one before)
  if (live)
#pragma unroll 8
    for (int t = t_begin; t < t_end; ++t) sum += hist[(int64_t)t * E + e];
  s_part[tid] = sum;
  __syncthreads();
  int run = 0, total_e = 0;
  if (live) {
    for (int p = 0; p < q; ++p) {
      const int v = s_part[p * E + e];
      if (p < part) run += v;
      total_e += v;
    }
#pragma unroll 8
    for (int t = t_begin; t < t_end; ++t) {
      const int64_t i = (int64_t)t * E + e;
      const int h = hist[i];
      tile_base[i] = run;
      run += h;
    }
  }
  int c = 0;
  if (live && part == 0) {
    routed[e] = total_e;
    c = total_e < C ? total_e : C;
    kept[e] = c;
  }
  int total;
  const int ex = block_exclusive_scan(c, smem, &total);
  if (live && part == 0) offsets[e] = pad ? e * C : ex;
  if (tid == 0) offsets[E] = pad ? E * C : total;
  for (int i = tid; i < k + 2; i += blockDim.x) drops[i] = 0;
  // padded experts own C rows each, which the GEMMs compute whole
  if (table)
    write_tile_table(live && part == 0 ? e : E, E, pad ? e * C : ex, pad ? C : c, bm, m_max,
                     smem, table);
}

__global__ void __launch_bounds__(kTileMax)
rank_kernel(const int32_t* __restrict__ idx, int64_t total, int64_t T, int te, int k, int E,
            int C, int nbits, bool slot_major, const int32_t* __restrict__ tile_base,
            const int32_t* __restrict__ offsets, int32_t* __restrict__ dest_row,
            int32_t* __restrict__ src_token, int32_t* __restrict__ src_slot,
            int32_t* __restrict__ drops, int64_t fill_R) {
  extern __shared__ int32_t sm[];
  constexpr int kWaves = kTileMax / kWave;
  int32_t* s_cnt = sm;                          // [kWaves][E] per-wave expert counts
  int32_t* s_tokdrop = sm + kWaves * E;         // [kTileMax] dropped slots per token
  int32_t* s_drop = s_tokdrop + kTileMax;       // [k + 2] block drop counters
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  // With fill_R > 0 the row slots [N, fill_R) past the kept rows get src_token = -1 here
  // (when no rows are copied, this saves the separate row kernel); kept rows are < N, so
  // no slot is written twice.
  if (fill_R > 0)
    for (int64_t r = offsets[E] + (int64_t)blockIdx.x * blockDim.x + tid; r < fill_R;
         r += (int64_t)gridDim.x * blockDim.x) {
      src_token[r] = -1;
      if (src_slot) src_slot[r] = -1;
    }
  for (int i = tid; i < kWaves * E; i += blockDim.x) s_cnt[i] = 0;
  s_tokdrop[tid] = 0;
  for (int i = tid; i < k + 2; i += blockDim.x) s_drop[i] = 0;
  __syncthreads();

  const int64_t p = (int64_t)blockIdx.x * te + tid;
  const bool active = tid < te && p < total;
  const int64_t f = active ? visit_entry(p, T, k, slot_major) : 0;  // entry t * k + j
  const int e = active ? idx[f] : -1;
  const bool valid = active && e >= 0 && e < E;

  // lanes of this wave holding the same expert: intersect the ballots of every id bit
  uint64_t same = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const uint64_t m = __ballot(bit);
    same &= bit ? m : ~m;
  }
  const int rank = __popcll(same & ((1ull << lane) - 1ull));
  if (valid && rank == 0) s_cnt[wave * E + e] = __popcll(same);
  __syncthreads();

  bool dropped = active;
  if (valid) {
    int pos = tile_base[(int64_t)blockIdx.x * E + e] + rank;
    for (int w = 0; w < wave; ++w) pos += s_cnt[w * E + e];
    const bool keep = pos < C;
    dropped = !keep;
    const int r = keep ? offsets[e] + pos : -1;
    dest_row[f] = r;
    if (keep) {
      src_token[r] = (int)(f / k);
      if (src_slot) src_slot[r] = (int)(f % k);
    }
  } else if (active) {
    dest_row[f] = -1;
  }
  if (dropped) {
    atomicAdd(&s_drop[0], 1);
    atomicAdd(&s_drop[1 + (int)(f % k)], 1);
    atomicAdd(&s_tokdrop[tid / k], 1);
  }
  __syncthreads();
  // token-major: the tile starts at a multiple of k, so token-local index is tid / k (the
  // slot-major count runs in token_drop_kernel)
  if (!slot_major && active && (tid % k) == 0 && s_tokdrop[tid / k] == k)
    atomicAdd(&s_drop[k + 1], 1);
  __syncthreads();
  for (int i = tid; i < k + 2; i += blockDim.x)
    if (s_drop[i]) atomicAdd(&drops[i], s_drop[i]);
}

// K3-K5 in one block of 1024 threads, for total <= kFusedPer * 1024 assignments and
// E <= kFusedDispatchMaxE experts (dispatch_fused).  Thread tid holds the experts of visit
// positions c * 1024 + tid (c < kFusedPer) in registers.  Pass 1 counts every expert in
// LDS; the block then scans the kept counts into offsets (and the tile table, when asked
// for); pass 2 walks the 1024-position chunks in visit order, ranking each assignment after
// the running count of its expert, the earlier waves of its chunk (per-wave counts in LDS)
// and the earlier lanes of its wave (ballots on the expert-id bits), the same positions the
// tiled kernels give.
// Drop counters and the per-token drop count live in LDS and are stored once at the end.
// Invalid expert ids (outside [0, E)) are ignored by the counts and dropped, as there.
constexpr int kFusedPer = (int)(kFusedDispatchEntries / 1024);
constexpr int kFusedWaves = 1024 / kWave;

__global__ void __launch_bounds__(1024)
dispatch_fused_kernel(const int32_t* __restrict__ idx, int total, int T, int k, int E, int C,
                      int nbits, bool slot_major, bool pad, int32_t* __restrict__ routed,
                      int32_t* __restrict__ kept, int32_t* __restrict__ offsets,
                      int32_t* __restrict__ dest_row, int32_t* __restrict__ src_token,
                      int32_t* __restrict__ src_slot, int32_t* __restrict__ drops,
                      int64_t fill_R, int32_t* __restrict__ table, int bm, int m_max) {
  extern __shared__ int32_t fsm[];
  int32_t* s_run = fsm;                      // [E] routed counts, then running positions
  int32_t* s_off = s_run + E;                // [E] first row of each expert
  int32_t* s_wc = s_off + E;                 // [kFusedWaves][E] per-wave counts of a chunk
  int32_t* s_tok = s_wc + kFusedWaves * E;   // [T] dropped assignments per token
  int32_t* s_drop = s_tok + T;               // [k + 2] drop counters
  __shared__ int smem[17];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  for (int i = tid; i < E; i += 1024) s_run[i] = 0;
  for (int i = tid; i < kFusedWaves * E; i += 1024) s_wc[i] = 0;
  for (int i = tid; i < T; i += 1024) s_tok[i] = 0;
  for (int i = tid; i < k + 2; i += 1024) s_drop[i] = 0;
  __syncthreads();
  // ev[c]: expert of visit position c * 1024 + tid; -1 an invalid id, -2 past the end
  int ev[kFusedPer];
#pragma unroll
  for (int c = 0; c < kFusedPer; ++c) {
    const int p = c * 1024 + tid;
    int e = -2;
    if (p < total) {
      e = idx[visit_entry(p, T, k, slot_major)];
      if (e < 0 || e >= E) e = -1;
    }
    ev[c] = e;
  }
#pragma unroll
  for (int c = 0; c < kFusedPer; ++c)
    if (ev[c] >= 0) atomicAdd(&s_run[ev[c]], 1);
  __syncthreads();
  // counts, capacity and offsets (E <= 256 threads hold one expert each)
  const int n_e = tid < E ? s_run[tid] : 0;
  const int c_e = n_e < C ? n_e : C;
  int n_kept;
  const int ex = block_exclusive_scan(c_e, smem, &n_kept);
  const int row0 = pad ? (tid < E ? tid * C : 0) : ex;
  if (tid < E) {
    routed[tid] = n_e;
    kept[tid] = c_e;
    offsets[tid] = row0;
    s_off[tid] = row0;
    s_run[tid] = 0;  // every thread has read its count (the scan holds barriers)
  }
  if (tid == 0) offsets[E] = pad ? E * C : n_kept;
  if (table) write_tile_table(tid < E ? tid : E, E, row0, pad ? C : c_e, bm, m_max, smem, table);
  // packed rows without a copy: the row slots past the kept rows are empty
  for (int64_t r = n_kept + tid; r < fill_R; r += 1024) {
    src_token[r] = -1;
    if (src_slot) src_slot[r] = -1;
  }
  __syncthreads();

  for (int c = 0; c < kFusedPer && c * 1024 < total; ++c) {
    const int p = c * 1024 + tid;
    const int e = ev[c];
    const bool valid = e >= 0, active = e != -2;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & ((1ull << lane) - 1ull));
    if (valid && rank == 0) s_wc[wave * E + e] = __popcll(same);
    __syncthreads();
    const int f = active ? (int)visit_entry(p, T, k, slot_major) : 0;  // entry t * k + j
    bool dropped = active;
    if (valid) {
      int pos = s_run[e] + rank;
      for (int w = 0; w < wave; ++w) pos += s_wc[w * E + e];
      const bool keep = pos < C;
      dropped = !keep;
      const int r = keep ? s_off[e] + pos : -1;
      dest_row[f] = r;
      if (keep) {
        src_token[r] = f / k;
        if (src_slot) src_slot[r] = f % k;
      }
    } else if (active) {
      dest_row[f] = -1;
    }
    if (dropped) {
      atomicAdd(&s_drop[0], 1);
      atomicAdd(&s_drop[1 + f % k], 1);
      atomicAdd(&s_tok[f / k], 1);
    }
    __syncthreads();
    // advance the running counts past this chunk and clear its wave counts
    for (int i = tid; i < E; i += 1024) {
      int add = 0;
      for (int w = 0; w < kFusedWaves; ++w) add += s_wc[w * E + i];
      s_run[i] += add;
    }
    __syncthreads();
    for (int i = tid; i < kFusedWaves * E; i += 1024) s_wc[i] = 0;
    __syncthreads();
  }
  // tokens whose k assignments were all dropped
  for (int t = tid; t < T; t += 1024)
    if (s_tok[t] == k) atomicAdd(&s_drop[k + 1], 1);
  __syncthreads();
  for (int i = tid; i < k + 2; i += 1024) drops[i] = s_drop[i];
}

// Tokens whose k assignments were all dropped, for the slot-major order (there a token's
// assignments lie in k different tiles of the rank kernel).
__global__ void __launch_bounds__(256)
token_drop_kernel(const int32_t* __restrict__ dest_row, int64_t T, int k,
                  int32_t* __restrict__ drops) {
  __shared__ int s_n;
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < T) {
    bool all = true;
    for (int j = 0; j < k; ++j) all = all && dest_row[t * k + j] < 0;
    if (all) atomicAdd(&s_n, 1);
  }
  __syncthreads();
  if (threadIdx.x == 0 && s_n) atomicAdd(&drops[k + 1], s_n);
}

// One wave per row, four rows per block, grid-stride over the R row slots (with x_perm
// null only the src_token entries of empty slots are written).  Packed rows:
// slots past N = offsets[E] only get src_token = -1.  Padded (C slots per expert): slot
// r belongs to expert r / C and is empty when r % C >= kept[r / C]; it gets src_token -1
// and a zero row.
__global__ void __launch_bounds__(256)
gather_rows_kernel(const char* __restrict__ x, int32_t* __restrict__ src_token,
                   int32_t* __restrict__ src_slot,
                   const int32_t* __restrict__ offsets, const int32_t* __restrict__ kept,
                   int E, int C, bool pad, int64_t R, int64_t row_bytes,
                   char* __restrict__ x_perm) {
  const int64_t N = offsets[E];
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int64_t nchunks = row_bytes / 16;
  for (int64_t r = (int64_t)blockIdx.x * 4 + wave; r < R; r += (int64_t)gridDim.x * 4) {
    if (pad) {
      if (r % C >= kept[r / C]) {
        if (lane == 0) {
          src_token[r] = -1;
          if (src_slot) src_slot[r] = -1;
        }
        if (!x_perm) continue;
        char* dst = x_perm + r * row_bytes;
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (int64_t c = lane; c < nchunks; c += kWave) st16(dst + c * 16, z);
        continue;
      }
    } else if (r >= N) {
      if (lane == 0) {
        src_token[r] = -1;
        if (src_slot) src_slot[r] = -1;
      }
      continue;
    }
    if (!x_perm) continue;  // tables only
    const int64_t t = src_token[r];
    const char* src = x + t * row_bytes;
    char* dst = x_perm + r * row_bytes;
    int64_t c = lane;
    for (; c + 3 * kWave < nchunks; c += 4 * kWave) {
      const u32x4 v0 = ld16(src + (c + 0 * kWave) * 16), v1 = ld16(src + (c + 1 * kWave) * 16);
      const u32x4 v2 = ld16(src + (c + 2 * kWave) * 16), v3 = ld16(src + (c + 3 * kWave) * 16);
      st16(dst + (c + 0 * kWave) * 16, v0);
      st16(dst + (c + 1 * kWave) * 16, v1);
      st16(dst + (c + 2 * kWave) * 16, v2);
      st16(dst + (c + 3 * kWave) * 16, v3);
    }
    for (; c < nchunks; c += kWave) st16(dst + c * 16, ld16(src + c * 16));
  }
}

// Observability: per-slot routed and kept counts, [k, E] each.  One thread per assignment
// adds into the global counters (up to 64 x 1024 of them, too many for an LDS histogram);
// integer adds make the result independent of their order.
__global__ void __launch_bounds__(256)
slot_counts_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ dest_row,
                   int64_t total, int k, int E, int32_t* __restrict__ routed_by_slot,
                   int32_t* __restrict__ kept_by_slot) {
  const int64_t f = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (f >= total) return;
  const int e = idx[f];
  if (e < 0 || e >= E) return;
  const int64_t c = (int64_t)(f % k) * E + e;
  atomicAdd(&routed_by_slot[c], 1);
  if (dest_row[f] >= 0) atomicAdd(&kept_by_slot[c], 1);
}

hipError_t launch_slot_counts(const int32_t* idx, const int32_t* dest_row, int64_t T,
                              int64_t k, int64_t E, int32_t* routed_by_slot,
                              int32_t* kept_by_slot, hipStream_t s) {
  hipError_t err;
  if ((err = launch_zero_i32(routed_by_slot, k * E, s)) != hipSuccess) return err;
  if ((err = launch_zero_i32(kept_by_slot, k * E, s)) != hipSuccess) return err;
  const int64_t total = T * k;
  if (total == 0) return hipSuccess;
  slot_counts_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
      idx, dest_row, total, (int)k, (int)E, routed_by_slot, kept_by_slot);
  return hipGetLastError();
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  const int64_t total = a.T * a.k;
  const int te = (int)dispatch_tile_entries(a.k);
  int ntiles = (int)dispatch_ntiles(a.T, a.k);
  int nbits = 0;
  while ((1ll << nbits) < a.E) ++nbits;
  hipError_t err;
  // packed rows without a copy: the rank kernel marks the empty row slots itself
  const bool tail_in_rank = !a.x_perm && !a.pad && ntiles > 0;
  const int bm = a.table ? a.table_bm : 0, m_max = a.table ? (int)a.table_m_max : 0;
  if (dispatch_fused(a.T, a.k, a.E)) {
    const size_t lds = ((2 + kFusedWaves) * a.E + a.T + a.k + 2) * sizeof(int32_t);
    dispatch_fused_kernel<<<1, 1024, lds, s>>>(
        a.topk_idx, (int)total, (int)a.T, (int)a.k, (int)a.E, (int)a.C, nbits, a.slot_major,
        a.pad, a.routed, a.kept, a.offsets, a.dest_row, a.src_token, a.src_slot, a.drops,
        tail_in_rank ? a.R : 0, a.table, bm, m_max);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    ntiles = 0;  // the tiled kernels below are not needed
  }
  if (ntiles > 0) {
    tile_hist_kernel<<<ntiles, kTileMax, a.E * sizeof(int32_t), s>>>(
        a.topk_idx, total, a.T, te, (int)a.k, (int)a.E, a.slot_major, a.tile_hist);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (total == 0 || ntiles > 0) {
    scan_kernel<<<1, 1024, 0, s>>>(a.tile_hist, ntiles, (int)a.E, (int)a.C, (int)a.k, a.pad,
                                   a.tile_base, a.routed, a.kept, a.offsets, a.drops, a.table,
                                   bm, m_max);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (ntiles > 0) {
    const size_t lds = ((kTileMax / kWave) * a.E + kTileMax + a.k + 2) * sizeof(int32_t);
    rank_kernel<<<ntiles, kTileMax, lds, s>>>(a.topk_idx, total, a.T, te, (int)a.k, (int)a.E,
                                              (int)a.C, nbits, a.slot_major, a.tile_base,
                                              a.offsets, a.dest_row, a.src_token,
                                              a.src_slot, a.drops,
                                              tail_in_rank ? a.R : 0);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (a.slot_major) {
      token_drop_kernel<<<(unsigned)((a.T + 255) / 256), 256, 0, s>>>(a.dest_row, a.T,
                                                                       (int)a.k, a.drops);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
  }
  if (a.R > 0 && !tail_in_rank) {
    int64_t blocks = (a.R + 3) / 4;
    if (blocks > 4096) blocks = 4096;
    gather_rows_kernel<<<(unsigned)blocks, 256, 0, s>>>(
        (const char*)a.x, a.src_token, a.src_slot, a.offsets, a.kept, (int)a.E, (int)a.C, a.pad,
        a.R, a.d * a.elt_bytes, (char*)a.x_perm);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
