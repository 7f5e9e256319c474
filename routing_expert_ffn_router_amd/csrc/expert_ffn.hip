// S6-S7: grouped SwiGLU expert FFN over the expert-contiguous rows of x_perm.
//
// [EP-serving] aiunderstanding.org, "Expert parallelism for MoE serving", sections "Deep
// dive" (each expert is a small feed-forward network) and "Technical details" (expert
// buffers keep the expert GEMMs regular); [EP-checks] airouter.kz, "Expert parallelism in
// MoE needs measurements before launch", section "All-to-all must be profiled separately
// from compute" (grouped GEMMs for the expert compute).  Layer specification:
//     h = silu(X Wg[e]^T) * (X Wu[e]^T)  (rounded to the storage type),  Y = h Wd[e]^T.
//
// One kernel template serves both GEMMs: C[rows of expert e, n] = A[rows] . B_e[n]^T with
// A and B both contiguous along the reduction axis (nn.Linear layout).
//   - Variable M per expert: the m-tiles of all experts are numbered consecutively and a
//     one-block kernel writes the table tile -> (expert, first row) on the device from the
//     expert offsets, so the host never waits for the routing.  The grid is sized from an
//     upper bound on the tile count and surplus blocks exit at once.
//   - Block tile BM x BN_W weight rows, K in 128-byte steps staged through LDS (two stages,
//     global loads of step k+1 in flight while step k is multiplied).  LDS rows are 128
//     bytes with the 16-byte chunks XOR-swizzled by (row & 7), so the MFMA fragment reads
//     (16 rows x one chunk column) hit distinct banks.
//   - SwiGLU: the B tile of a wave holds NT/2 tiles of gate rows followed by the NT/2 tiles
//     of up rows for the same output columns, so gate and up accumulators of one output
//     element sit in the same lane and the epilogue computes silu(g) * u in registers.
//   - Block order: blocks are dealt round-robin to the 8 XCDs; the logical tile index is
//     remapped so each XCD walks a contiguous range in which neighbouring tiles share the
//     A rows (same m-tile) and the B rows (same n-group), keeping both in that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace moe {

__device__ inline float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

template <int WAVES_M, int WAVES_N, int MT, int NT, bool SWIGLU>
struct GemmShape {
  static constexpr int kThreads = WAVES_M * WAVES_N * kWave;
  static constexpr int BM = WAVES_M * MT * 16;
  static constexpr int kWaveRows = NT * 16;             // weight rows per wave
  static constexpr int BNW = WAVES_N * kWaveRows;       // weight rows per block
  static constexpr int BN = SWIGLU ? BNW / 2 : BNW;     // output columns per block
  // 16-byte chunks per thread and stage (A: the last round may leave threads idle)
  static constexpr int kAChunks = (BM * 8 + kThreads - 1) / kThreads;
  static constexpr bool kAPartial = BM * 8 % kThreads != 0;
  static constexpr int kBChunks = BNW * 8 / kThreads;
  static constexpr int kStageBytes = (BM + BNW) * 128;
  static_assert(BNW * 8 % kThreads == 0, "tile / thread mismatch");
  static_assert(!SWIGLU || NT % 2 == 0, "SwiGLU needs gate and up halves");
};

// Tile table for one row-tile height BM: table[0] = number of m-tiles over all experts;
// entry i (i < table[0]) is (expert, first row) at table[1 + 2i], table[2 + 2i].  Experts
// are numbered in index order and their tiles in row order.
__global__ void __launch_bounds__(1024)
tile_table_kernel(const int32_t* __restrict__ offsets, int E, int bm, int m_max,
                  int32_t* __restrict__ table) {
  __shared__ int smem[17];
  __shared__ int s_pre[1024];
  __shared__ int s_cnt[1024];
  const int e = threadIdx.x;
  const int c = e < E ? offsets[e + 1] - offsets[e] : 0;
  const int tiles = (c + bm - 1) / bm;
  int total;
  const int pre = block_exclusive_scan(tiles, smem, &total);
  if (e < E) {
    s_pre[e] = pre;
    s_cnt[e] = tiles;
  }
  if (threadIdx.x == 0) table[0] = total < m_max ? total : m_max;
  __syncthreads();
  for (int x = 0; x < E; ++x) {
    const int n = s_cnt[x], p0 = s_pre[x], row0 = offsets[x];
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      if (p0 + i >= m_max) break;
      table[1 + 2 * (p0 + i)] = x;
      table[2 + 2 * (p0 + i)] = row0 + i * bm;
    }
  }
}

template <class T, int WAVES_M, int WAVES_N, int MT, int NT, bool SWIGLU>
__global__ void __launch_bounds__(WAVES_M* WAVES_N* kWave)
grouped_gemm_kernel(const T* __restrict__ A, const T* __restrict__ B0,
                    const T* __restrict__ B1, int64_t b_expert_stride, T* __restrict__ C,
                    int K, int N_out, const int32_t* __restrict__ offsets,
                    const int32_t* __restrict__ table, int m_tiles_max, int n_tiles,
                    int group_n, int grid_logical) {
  using S = GemmShape<WAVES_M, WAVES_N, MT, NT, SWIGLU>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  // ---- block -> (expert, m-tile, n-tile) ------------------------------------------------
  const int bid = blockIdx.x;
  const int per_xcd = gridDim.x >> 3;
  const int logical = (bid & 7) * per_xcd + (bid >> 3);
  if (logical >= grid_logical) return;
  const int per_group = m_tiles_max * group_n;
  const int grp = logical / per_group, rem = logical - grp * per_group;
  const int mt = rem / group_n, nt = grp * group_n + (rem - (rem / group_n) * group_n);
  if (nt >= n_tiles) return;
  if (mt >= table[0]) return;
  const int e = table[1 + 2 * mt];
  const int m_begin = table[2 + 2 * mt];
  const int m_end = offsets[e + 1];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int64_t row_bytes = (int64_t)K * sizeof(T);

  // ---- per-thread global source rows (fixed over k) ---------------------------------------
  const char* a_src[S::kAChunks];
  int a_lds[S::kAChunks];
#pragma unroll
  for (int i = 0; i < S::kAChunks; ++i) {
    const int c0 = tid + i * S::kThreads;
    const int c = (S::kAPartial && c0 >= S::BM * 8) ? c0 % (S::BM * 8) : c0;  // duplicate load
    const int r = c >> 3, ch = c & 7;
    const int gr = min(m_begin + r, m_end - 1);  // rows past the expert: computed, not stored
    a_src[i] = reinterpret_cast<const char*>(A) + (int64_t)gr * row_bytes + ch * 16;
    a_lds[i] = r * 128 + ((ch ^ (r & 7)) << 4);
  }
  const char* b_src[S::kBChunks];
  int b_lds[S::kBChunks];
  const T* B0e = B0 + (int64_t)e * b_expert_stride;
  const T* B1e = SWIGLU ? B1 + (int64_t)e * b_expert_stride : nullptr;
#pragma unroll
  for (int i = 0; i < S::kBChunks; ++i) {
    const int c = tid + i * S::kThreads, r = c >> 3, ch = c & 7;
    const T* rowp;
    if (SWIGLU) {
      const int w = r / S::kWaveRows, within = r % S::kWaveRows, half = S::kWaveRows / 2;
      // columns past N_out (last n-tile) are clamped: computed, never stored
      const int col = min(nt * S::BN + w * half + (within % half), N_out - 1);
      rowp = (within < half ? B0e : B1e) + (int64_t)col * K;
    } else {
      rowp = B0e + (int64_t)min(nt * S::BN + r, N_out - 1) * K;
    }
    b_src[i] = reinterpret_cast<const char*>(rowp) + ch * 16;
    b_lds[i] = S::BM * 128 + r * 128 + ((ch ^ (r & 7)) << 4);
  }

  f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[S::kAChunks], rb[S::kBChunks];
  auto load_global = [&](int kt) {
    const int64_t off = (int64_t)kt * 128;
#pragma unroll
    for (int i = 0; i < S::kAChunks; ++i) ra[i] = ld16(a_src[i] + off);
#pragma unroll
    for (int i = 0; i < S::kBChunks; ++i) rb[i] = ld16(b_src[i] + off);
  };
  auto store_lds = [&](int stage) {
    char* base = smem + stage * S::kStageBytes;
#pragma unroll
    for (int i = 0; i < S::kAChunks; ++i) st16(base + a_lds[i], ra[i]);
#pragma unroll
    for (int i = 0; i < S::kBChunks; ++i) st16(base + b_lds[i], rb[i]);
  };

  // fragment addresses: row (lane & 15) of each 16-row tile, chunk (ks * 4 + lane / 16)
  // swizzled by (row & 7) == (lane & 7)
  const int frag_row = lane & 15, frag_grp = lane >> 4, swz = lane & 7;
  const int a_frag = (wm * MT * 16 + frag_row) * 128;
  const int b_frag = S::BM * 128 + (wn * NT * 16 + frag_row) * 128;

  auto compute = [&](int stage) {
    const char* base = smem + stage * S::kStageBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int chunk_off = ((ks * 4 + frag_grp) ^ swz) << 4;
      u32x4 fa[MT], fb[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i) fa[i] = ld16(base + a_frag + i * 16 * 128 + chunk_off);
#pragma unroll
      for (int j = 0; j < NT; ++j) fb[j] = ld16(base + b_frag + j * 16 * 128 + chunk_off);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) mma_chunk(acc[i][j], fa[i], fb[j], T());
    }
  };

  const int KT = (int)(row_bytes / 128);
  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    if (more) load_global(kt + 1);
    compute(kt & 1);
    if (more) store_lds((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue ----------------------------------------------------------------------------
  constexpr int NOUT = SWIGLU ? NT / 2 : NT;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m_begin + wm * MT * 16 + i * 16 + frag_grp * 4 + r;
      if (row >= m_end) continue;
      const int col0 = nt * S::BN + wn * NOUT * 16 + frag_row;
      T* crow = C + (int64_t)row * N_out + col0;
#pragma unroll
      for (int j = 0; j < NOUT; ++j) {
        if (col0 + j * 16 >= N_out) continue;
        float v;
        if (SWIGLU)
          v = silu_f32(acc[i][j][r]) * acc[i][j + NOUT][r];
        else
          v = acc[i][j][r];
        crow[j * 16] = Elt<T>::from_f32(v);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Prefill-sized experts: 256 x 256 block tile, 8 waves, 32x32 MFMA tiles, 4-stage LDS
// pipeline fed by direct global -> LDS loads (global_load_lds_dwordx4).
//
// Each stage holds 32 reduction elements (64 bytes) of the block's 256 A rows and 256
// weight rows: 512 LDS rows of 64 bytes = 32 KB; four stages use 128 KB of the CU's 160 KB.
// A wave's direct-load instruction writes 64 lanes x 16 bytes = 16 consecutive LDS rows,
// lane L landing at row L / 4, slot L % 4 of them.  The slot holding k-chunk c of row r is
// c ^ ((r >> 2) & 3).  A 32x32 fragment read (32 rows at one chunk position in each half
// of the wave) then runs at the full LDS rate of gfx950: measured 4.75 cycles per 64-lane
// 16-byte read on one CU with 8 waves, against 16.2 without a swizzle.  The lane therefore
// fetches chunk (L % 4) ^ ((r >> 2) & 3).
//
// Pipeline: stages k+1 and k+2 are in flight while stage k is multiplied; at the top of
// step k a wave waits until its own loads of stage k have landed (vmcnt counts the 4
// direct loads per wave per stage) and a barrier makes every wave's loads visible; then
// stage k+3 is issued into the buffer that step k-1 just finished reading.  The stage
// buffers are distinct __restrict__ pointers of an inlined function so the compiler keeps
// these explicit waits instead of inserting a full wait before every LDS read.
//
// Waves form a 2 (rows) x 4 (weight rows) grid; each owns 128 x 64 of the tile (4 x 2
// MFMA tiles of 32 x 32).  With SwiGLU a wave's 64 weight rows are 32 gate rows followed
// by the 32 up rows of the same output columns, so a block produces 256 x 128 of h.
// ---------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) char lds_char;
typedef const __attribute__((address_space(1))) void gbl_void;

// ROWB: bytes of each row per stage (64 or 128); STAGES: LDS stages (4 or 2).
template <int ROWB, int STAGES>
struct PrefillTileT {
  static constexpr int BM = 256, BNW = 256, kWaves = 8, kThreads = 512;
  static constexpr int WM = 2, WN = 4, MT = 4, NT = 2;  // 32x32 tiles per wave
  static constexpr int kRowBytes = ROWB;
  static constexpr int kChunks = ROWB / 16;                  // 16-byte chunks per row
  static constexpr int kKSteps = ROWB / 32;                  // 32-byte MFMA k-steps
  static constexpr int kStageBytes = (BM + BNW) * kRowBytes;
  static constexpr int kStages = STAGES;
  static constexpr int kRowsPerLoad = 1024 / ROWB;           // rows per direct load
  static constexpr int kDmaPerWave = (BM + BNW) / kRowsPerLoad / kWaves;
  // slot of k-chunk c in row r: c ^ swz(r); conflict-free 32x32 fragment reads (measured)
  __device__ static inline int swz(int r) {
    return ROWB == 64 ? ((r >> 2) & 3) : ((r >> 1) & 7);
  }
};
using PrefillTile = PrefillTileT<128, 2>;

// wait until at most N direct loads of this wave are outstanding, then block barrier
template <int N>
__device__ inline void wait_vm_barrier() {
  static_assert(N == 0 || N == 4 || N == 8 || N == 16, "vmcnt immediate");
  if (N == 16)
    asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  else if (N == 8)
    asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  else if (N == 4)
    asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

template <class T, bool SWIGLU, class P>
__device__ __attribute__((always_inline)) inline void prefill_gemm_body(
    const T* __restrict__ A, const T* __restrict__ B0, const T* __restrict__ B1,
    int64_t b_expert_stride, T* __restrict__ C, int K, int N_out,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ table,
    int m_tiles_max, int n_tiles, int group_n, int grid_logical, lds_char* __restrict__ s0,
    lds_char* __restrict__ s1, lds_char* __restrict__ s2, lds_char* __restrict__ s3) {
  constexpr int BN = SWIGLU ? P::BNW / 2 : P::BNW;
  const int bid = blockIdx.x;
  const int per_xcd = gridDim.x >> 3;
  const int logical = (bid & 7) * per_xcd + (bid >> 3);
  if (logical >= grid_logical) return;
  const int per_group = m_tiles_max * group_n;
  const int grp = logical / per_group, rem = logical - grp * per_group;
  const int mt = rem / group_n, nt = grp * group_n + (rem - (rem / group_n) * group_n);
  if (nt >= n_tiles) return;
  if (mt >= table[0]) return;
  const int e = table[1 + 2 * mt];
  const int m_begin = table[2 + 2 * mt];
  const int m_end = offsets[e + 1];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int wm = wave / P::WN, wn = wave % P::WN;
  const int64_t row_bytes = (int64_t)K * sizeof(T);

  // per-lane source of each direct load (k offset 0); LDS row of load i of this wave:
  // (wave * kDmaPerWave + i) * 16 + lane / 4
  const char* src[P::kDmaPerWave];
  const T* B0e = B0 + (int64_t)e * b_expert_stride;
  const T* B1e = SWIGLU ? B1 + (int64_t)e * b_expert_stride : nullptr;
#pragma unroll
  for (int i = 0; i < P::kDmaPerWave; ++i) {
    const int r = (wave * P::kDmaPerWave + i) * P::kRowsPerLoad + lane / P::kChunks;
    const int c = (lane % P::kChunks) ^ P::swz(r);
    const char* rowp;
    if (r < P::BM) {
      const int gr = min(m_begin + r, m_end - 1);  // rows past the expert: never stored
      rowp = reinterpret_cast<const char*>(A) + (int64_t)gr * row_bytes;
    } else {
      const int br = r - P::BM;
      if (SWIGLU) {
        const int w = br / 64, within = br % 64;
        const int col = min(nt * BN + w * 32 + (within % 32), N_out - 1);
        rowp = reinterpret_cast<const char*>((within < 32 ? B0e : B1e) + (int64_t)col * K);
      } else {
        rowp = reinterpret_cast<const char*>(B0e + (int64_t)min(nt * BN + br, N_out - 1) * K);
      }
    }
    src[i] = rowp + c * 16;
  }
  const int dma_lds = wave * P::kDmaPerWave * 1024;

  f32x16 acc[P::MT][P::NT];
#pragma unroll
  for (int i = 0; i < P::MT; ++i)
#pragma unroll
    for (int j = 0; j < P::NT; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // a wave whose 128-row band lies past the expert's rows skips its MFMAs
  const bool band_live = m_begin + wm * P::MT * 32 < m_end;
  const int frag_row = lane & 31, frag_half = lane >> 5;
  const int a_frag = (wm * P::MT * 32 + frag_row) * P::kRowBytes;
  const int b_frag = (P::BM + wn * P::NT * 32 + frag_row) * P::kRowBytes;
  const int swz = P::swz(frag_row);

  auto issue = [&](int kt, lds_char* buf) {
    const int64_t koff = (int64_t)kt * P::kRowBytes;
#pragma unroll
    for (int i = 0; i < P::kDmaPerWave; ++i)
      __builtin_amdgcn_global_load_lds((gbl_void*)(src[i] + koff), buf + dma_lds + i * 1024, 16,
                                       0, 0);
  };
  // Fragments of one 32-byte k-step: 4 A tiles + 2 B tiles.  The reads of k-step s+1 are
  // issued before the MFMAs of k-step s (two register sets), and the scheduling groups
  // pin that order, so each k-step's 8 MFMAs cover the next k-step's LDS latency.
  auto load_frags = [&](const lds_char* buf, int ks, u32x4* fa, u32x4* fb) {
    const int slot = ((ks * 2 + frag_half) ^ swz) << 4;
#pragma unroll
    for (int j = 0; j < P::NT; ++j)
      fb[j] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          buf + b_frag + j * 32 * P::kRowBytes + slot);
#pragma unroll
    for (int i = 0; i < P::MT; ++i)
      fa[i] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          buf + a_frag + i * 32 * P::kRowBytes + slot);
  };
  auto compute = [&](const lds_char* buf) {
    if (!band_live) return;
    u32x4 fa[2][P::MT], fb[2][P::NT];
    load_frags(buf, 0, fa[0], fb[0]);
#pragma unroll
    for (int ks = 0; ks < P::kKSteps; ++ks) {
      if (ks + 1 < P::kKSteps) load_frags(buf, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < P::MT; ++i)
#pragma unroll
        for (int j = 0; j < P::NT; ++j)
          mma32_chunk(acc[i][j], fa[ks & 1][i], fb[ks & 1][j], T());
      // order: [6 LDS reads of step 0] then per step: 6 reads of the next step, 8 MFMAs
      if (ks == 0) __builtin_amdgcn_sched_group_barrier(0x100, P::MT + P::NT, 0);
      if (ks + 1 < P::kKSteps) __builtin_amdgcn_sched_group_barrier(0x100, P::MT + P::NT, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, P::MT * P::NT, 0);
    }
  };
  const int KT = (int)(row_bytes / P::kRowBytes);
  constexpr int D = P::kStages - 1;  // stages in flight ahead of the one multiplied
  auto step = [&](int kt, const lds_char* cur, lds_char* nxt) {
    if (kt >= KT) return;
    // stage kt must have landed; stages kt+1 .. kt+D-1 may still be in flight
    if (D >= 3 && kt + 2 < KT)
      wait_vm_barrier<2 * P::kDmaPerWave * (D >= 3)>();
    else if (D >= 2 && kt + 1 < KT)
      wait_vm_barrier<P::kDmaPerWave * (D >= 2)>();
    else
      wait_vm_barrier<0>();
    if (kt + D < KT) issue(kt + D, nxt);
    compute(cur);
  };

  if (P::kStages == 4) {
    issue(0, s0);
    if (KT > 1) issue(1, s1);
    if (KT > 2) issue(2, s2);
    for (int kt = 0; kt < KT; kt += 4) {
      step(kt + 0, s0, s3);
      step(kt + 1, s1, s0);
      step(kt + 2, s2, s1);
      step(kt + 3, s3, s2);
    }
  } else {
    issue(0, s0);
    for (int kt = 0; kt < KT; kt += 2) {
      step(kt + 0, s0, s1);
      step(kt + 1, s1, s0);
    }
  }

  if (!band_live) return;
  // lane holds column (lane % 32) and rows 8 * (q / 4) + 4 * (lane / 32) + q % 4 of a tile
  constexpr int NOUT = SWIGLU ? P::NT / 2 : P::NT;
#pragma unroll
  for (int i = 0; i < P::MT; ++i) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = m_begin + wm * P::MT * 32 + i * 32 + 8 * (q >> 2) + 4 * frag_half + (q & 3);
      if (row >= m_end) continue;
      const int col0 = nt * BN + wn * NOUT * 32 + frag_row;
      T* crow = C + (int64_t)row * N_out + col0;
#pragma unroll
      for (int j = 0; j < NOUT; ++j) {
        if (col0 + j * 32 >= N_out) continue;
        float v;
        if (SWIGLU)
          v = silu_f32(acc[i][j][q]) * acc[i][j + NOUT][q];
        else
          v = acc[i][j][q];
        crow[j * 32] = Elt<T>::from_f32(v);
      }
    }
  }
}

template <class T, bool SWIGLU>
__global__ void __launch_bounds__(PrefillTile::kThreads)
prefill_gemm_kernel(const T* __restrict__ A, const T* __restrict__ B0,
                    const T* __restrict__ B1, int64_t b_expert_stride, T* __restrict__ C, int K,
                    int N_out, const int32_t* __restrict__ offsets,
                    const int32_t* __restrict__ table, int m_tiles_max, int n_tiles,
                    int group_n, int grid_logical) {
  extern __shared__ __attribute__((aligned(1024))) char smem_dyn[];
  lds_char* base = (lds_char*)smem_dyn;
  constexpr int S = PrefillTile::kStageBytes;
  // with two stages, s2 and s3 are never used
  prefill_gemm_body<T, SWIGLU, PrefillTile>(
      A, B0, B1, b_expert_stride, C, K, N_out, offsets, table, m_tiles_max, n_tiles, group_n,
      grid_logical, base, base + S, base + (PrefillTile::kStages > 2 ? 2 * S : 0),
      base + (PrefillTile::kStages > 3 ? 3 * S : 0));
}

// ---------------------------------------------------------------------------------------
// launch configurations
// ---------------------------------------------------------------------------------------
// Row-tile heights: prefill-sized experts (mean > 32 rows) use the 256-row prefill kernel,
// decode-sized ones 16-row tiles.
FfnPlan ffn_plan(int64_t T, int64_t E, int64_t k, int64_t C, int64_t R) {
  FfnPlan p;
  p.small = T * k <= 32 * E;
  p.bm = p.small ? 16 : PrefillTile::BM;
  int64_t m_max = (R + E * (p.bm - 1)) / p.bm;
  const int64_t m_cap = E * ((C + p.bm - 1) / p.bm);
  p.m_max = m_cap < m_max ? m_cap : m_max;
  if (p.m_max < 0) p.m_max = 0;
  return p;
}

namespace {

template <class T, int WM, int WN, int MT, int NT, bool SW>
hipError_t launch_gemm(const T* A, const T* B0, const T* B1, int64_t b_stride, T* C, int K,
                       int N_out, const int32_t* offsets, const int32_t* table, int64_t m_max,
                       hipStream_t s) {
  using S = GemmShape<WM, WN, MT, NT, SW>;
  if (m_max <= 0) return hipSuccess;
  const int n_tiles = (N_out + S::BN - 1) / S::BN;
  const int group_n = n_tiles < 8 ? n_tiles : 8;
  const int n_groups = (n_tiles + group_n - 1) / group_n;
  const int64_t logical = m_max * group_n * n_groups;
  const int64_t grid = (logical + 7) / 8 * 8;
  const size_t lds = 2 * S::kStageBytes;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)grouped_gemm_kernel<T, WM, WN, MT, NT, SW>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  grouped_gemm_kernel<T, WM, WN, MT, NT, SW><<<(unsigned)grid, S::kThreads, lds, s>>>(
      A, B0, B1, b_stride, C, K, N_out, offsets, table, (int)m_max, n_tiles, group_n,
      (int)logical);
  return hipGetLastError();
}

template <class T, bool SW>
hipError_t launch_prefill(const T* A, const T* B0, const T* B1, int64_t b_stride, T* C, int K,
                          int N_out, const int32_t* offsets, const int32_t* table,
                          int64_t m_max, hipStream_t s) {
  using P = PrefillTile;
  if (m_max <= 0) return hipSuccess;
  constexpr int BN = SW ? P::BNW / 2 : P::BNW;
  const int n_tiles = (N_out + BN - 1) / BN;
  const int group_n = n_tiles < 8 ? n_tiles : 8;
  const int n_groups = (n_tiles + group_n - 1) / group_n;
  const int64_t logical = m_max * group_n * n_groups;
  const int64_t grid = (logical + 7) / 8 * 8;
  const size_t lds = (size_t)P::kStages * P::kStageBytes;
  hipError_t e = hipFuncSetAttribute((const void*)prefill_gemm_kernel<T, SW>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  prefill_gemm_kernel<T, SW><<<(unsigned)grid, P::kThreads, lds, s>>>(
      A, B0, B1, b_stride, C, K, N_out, offsets, table, (int)m_max, n_tiles, group_n,
      (int)logical);
  return hipGetLastError();
}

hipError_t launch_table(const FfnArgs& a, const FfnPlan& p, hipStream_t s) {
  if (p.m_max <= 0) return hipSuccess;
  tile_table_kernel<<<1, 1024, 0, s>>>(a.offsets, (int)a.E, p.bm, (int)p.m_max, a.sched);
  return hipGetLastError();
}

template <class T>
hipError_t run_gate_up(const FfnArgs& a, const FfnPlan& p, hipStream_t s) {
  const T* xp = (const T*)a.x_perm;
  T* h = (T*)a.h;
  const int64_t stride = a.F * a.d;
  if (p.small)
    return launch_gemm<T, 1, 4, 1, 8, true>(xp, (const T*)a.w_gate, (const T*)a.w_up, stride,
                                            h, (int)a.d, (int)a.F, a.offsets, a.sched,
                                            p.m_max, s);
  return launch_prefill<T, true>(xp, (const T*)a.w_gate, (const T*)a.w_up, stride, h,
                                 (int)a.d, (int)a.F, a.offsets, a.sched, p.m_max, s);
}

template <class T>
hipError_t run_down(const FfnArgs& a, const FfnPlan& p, hipStream_t s) {
  const T* h = (const T*)a.h;
  T* y = (T*)a.y_perm;
  const int64_t stride = a.d * a.F;
  if (p.small)
    return launch_gemm<T, 1, 4, 1, 8, false>(h, (const T*)a.w_down, nullptr, stride, y,
                                             (int)a.F, (int)a.d, a.offsets, a.sched, p.m_max,
                                             s);
  return launch_prefill<T, false>(h, (const T*)a.w_down, nullptr, stride, y, (int)a.F,
                                  (int)a.d, a.offsets, a.sched, p.m_max, s);
}

}  // namespace

hipError_t launch_expert_ffn(const FfnArgs& a, int which, hipStream_t s) {
  if (a.R <= 0) return hipSuccess;
  const FfnPlan p = ffn_plan(a.T, a.E, a.k, a.C, a.R);
  hipError_t err = launch_table(a, p, s);
  if (err != hipSuccess) return err;
  if (which & 1) {
    err = a.dtype == 1 ? run_gate_up<bf16>(a, p, s) : run_gate_up<float>(a, p, s);
    if (err != hipSuccess) return err;
  }
  if (which & 2) err = a.dtype == 1 ? run_down<bf16>(a, p, s) : run_down<float>(a, p, s);
  return err;
}

}  // namespace moe
