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
//   - Operands reach LDS by direct buffer -> LDS loads in 128-byte row pieces, in a ring of
//     stages; fragments are read with a measured bank-conflict-free swizzle and fed to
//     16x16x32 MFMAs in the bf16 prefill tiles (on random data they hold a higher clock under
//     the power limit than the 32x32x16 form) and 32x32x16 MFMAs in the decode tiles and
//     in fp32.
//   - Tile shapes of the same template: prefill-sized experts (mean > 32 rows) use
//     256 x 256 tiles (128 flop per loaded byte) or, when that needs fewer row tiles or
//     pads fewer rows, 320 x 256 tiles (142 flop per byte), an expert's short last tile
//     128 x 256, or 128 x 512 (two n-tiles) behind two or more full 320-row tiles so that it
//     keeps their pace through the shared weight panel; decode-sized experts stream
//     weights in three stages with 64 x 256 tiles for gate/up (80 KB of weight reads in
//     flight per CU) and 64 x 128 tiles for down (two blocks per CU).
//   - A wave band that ends inside an expert's last rows skips the MFMAs of its empty
//     32-row tiles (a copy of the k-loop per live-tile count).
//   - SwiGLU: the gate and up rows of the same output columns are loaded side by side, so
//     the gate and up accumulators of one output element sit in the same lane and the
//     epilogue computes silu(g) * u in registers.
//   - Epilogue: the accumulators hold the transposed tile (weight fragment first), so each
//     lane writes 4 consecutive outputs into LDS; the block then stores its tile from LDS
//     with 16-byte stores over whole cache lines.
//   - Block order: blocks are dealt round-robin to the 8 XCDs; the logical tile index is
//     remapped so each XCD walks a contiguous range in which neighbouring tiles share the
//     A rows (same m-tile) and the B rows (same n-group), keeping both in that XCD's L2.
//     The n-group width comes from the launch plan.
//   - Weights that each tile reads alone (at most two row tiles per expert) are loaded with
//     the non-temporal hint, so they do not displace the shared activation rows.
//   - A down GEMM with few, long tiles runs the tiles of its last, partial round in up to 8
//     pieces along the reduction, whose fp32 partial sums a second launch adds in a fixed
//     order (deterministic), so that round does not leave most CUs idle (tail split).
//   - Dense mode (no tile table, fp32 output with a column bias) serves the router logits
//     of shapes with many tokens and experts.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace moe {

// silu(g) = g / (1 + e^-g) with the hardware reciprocal (about 1 ulp) instead of a correctly
// rounded division: the SwiGLU epilogue evaluates it for every output of the gate/up GEMM,
// and the division's ten instructions made that epilogue several percent of a tile.  For
// g < -88 the reciprocal of +inf gives -0.0 where the exact value is below 1e-36.
__device__ inline float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Tile table for one row-tile height BM: table[0] = number of m-tiles over all experts;
// entry i (i < table[0]) is (expert, first row) at table[1 + 2i], table[2 + 2i].  Experts
// are numbered in index order and their tiles in row order.
__global__ void __launch_bounds__(1024)
tile_table_kernel(const int32_t* __restrict__ offsets, int E, int bm, int m_max,
                  int32_t* __restrict__ table) {
  __shared__ int smem[17];
  const int e = threadIdx.x;
  const int row0 = e < E ? offsets[e] : 0;
  const int c = e < E ? offsets[e + 1] - row0 : 0;
  const int tiles = (c + bm - 1) / bm;
  int total;
  const int pre = block_exclusive_scan(tiles, smem, &total);
  if (threadIdx.x == 0) table[0] = total < m_max ? total : m_max;
  // each thread writes its own expert's tiles (E <= 1024 = blockDim)
  for (int i = 0; i < tiles && pre + i < m_max; ++i) {
    table[1 + 2 * (pre + i)] = e;
    table[2 + 2 * (pre + i)] = row0 + i * bm;
  }
}

// ---------------------------------------------------------------------------------------
// Block tile GEMM: 8 waves, 32x32 MFMA tiles, a ring of LDS stages fed by direct
// buffer -> LDS loads (buffer_load_dwordx4 ... lds).
//
// A stage holds ROWB bytes of the reduction axis of each of the tile's rows: first the BM
// activation rows, then the weight rows (with SwiGLU the BNW/2 gate rows, then the BNW/2
// up rows of the same output columns).  One direct load writes 64 lanes x 16 bytes, i.e.
// 1024 / ROWB consecutive LDS rows, lane L landing at row L / (ROWB/16), slot
// L % (ROWB/16).  The slot holding k-chunk c of row r is c ^ swz(r); the lane therefore
// fetches chunk (L % (ROWB/16)) ^ swz(r).  With this swizzle a 32x32 fragment read (32
// rows at one chunk position in each half of the wave) runs at the full LDS rate of gfx950
// (measured 4.75 cycles per 64-lane 16-byte read on one CU with 8 waves, against 16.2
// without it).  Row pieces of 128 bytes (whole cache lines) measured clearly faster than
// 64-byte pieces with more stages.
//
// Pipeline: STAGES - 1 stages are in flight while one is multiplied.  At the top of step k
// a wave waits until its own loads of stage k have landed (vmcnt counts its direct loads)
// and a barrier makes every wave's loads visible; then stage k + STAGES - 1 is issued into
// the buffer that step k-1 finished reading.  The stage buffers are distinct __restrict__
// pointers of an inlined function so the compiler keeps these explicit waits instead of
// inserting a full wait before every LDS read.
//
// Waves form a WM (rows) x WN (weight rows) grid; wave (wm, wn) owns BM/WM activation rows
// and BNW/WN weight rows (MT x NT MFMA tiles).  With SwiGLU the wave's weight rows are
// NT/2 tiles of gate rows and the NT/2 tiles of up rows of the same output columns, so
// the gate and up accumulators of one output element sit in the same lane.
// ---------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) char lds_char;

// ROWB: bytes of each row per stage (64 or 128); STAGES: LDS stages (2, 3 or 4);
// BM_ activation rows and BNW_ weight rows per block; the 8 waves split it WM_ x WN_.
// DSEL_: which waves issue the direct loads: 0 = all eight; 1 = waves 4-7, one per SIMD
// (waves are placed on the SIMDs round-robin), so each SIMD keeps one wave that never
// waits on the address unit (measured about 2.5% faster on the prefill tiles).
// M16_: each 32x32 tile of a wave is computed as 2 x 2 tiles of v_mfma_f32_16x16x32_bf16
// (64-byte k-steps) instead of v_mfma_f32_32x32x16_bf16 (32-byte k-steps).  Same results;
// on random data the 16x16 form holds a higher clock under the power limit (measured by
// the calibration loop: 1.94 against 1.75 GHz), but its fragments need twice the registers
// per k-step: the 320-row tile runs the lean fragment schedule (kLean).  M16_ = 2: the
// 16x16 form for bf16 only (ForElt); fp32 gains nothing from it and would run short of
// registers.
template <int ROWB, int STAGES, int BM_, int BNW_, int WM_, int WN_, int DSEL_ = 0,
          int BSTAGES_ = 0, int M16_ = 0>
struct PrefillTileT {
  static constexpr int BM = BM_, BNW = BNW_, kWaves = 8, kThreads = 512;
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int kDmaSel = DSEL_;
  static constexpr int kDmaWaves = DSEL_ == 0 ? 8 : 4;
  static constexpr int MT = BM / WM / 32, NT = BNW / WN / 32;  // 32x32 tiles per wave
  static constexpr int kWaveCols = NT * 32;                    // weight rows per wave
  static constexpr int kRowBytes = ROWB;
  static constexpr int kChunks = ROWB / 16;                  // 16-byte chunks per row
  static constexpr bool kM16 = M16_ != 0;
  // 16x16 form with more than four 32-row tiles per wave: the lean fragment schedule
  // (compute_lean), whose fragments fit the registers the 320-row tile leaves
  static constexpr bool kLean = kM16 && BM_ / WM_ / 32 > 4;
  static constexpr int kSub = kM16 ? 2 : 1;          // MFMA tiles per 32 rows (and columns)
  static constexpr int kFragRows = 32 / kSub;        // rows of one MFMA operand fragment
  static constexpr int kStepChunks = 64 / kFragRows;  // 16-byte chunks of one k-step
  static constexpr int kKSteps = ROWB / 16 / kStepChunks;  // MFMA k-steps per stage
  // separate rings: activation rows (kAStages) and weight rows (kBStages)
  static constexpr int kAStages = STAGES, kBStages = BSTAGES_ ? BSTAGES_ : STAGES;
  static constexpr int kABytes = BM * kRowBytes, kBBytes = BNW * kRowBytes;
  static constexpr int kLdsBytes = kAStages * kABytes + kBStages * kBBytes;
  static constexpr int kRowsPerLoad = 1024 / ROWB;           // rows per direct load
  static constexpr int kALoads = BM / kRowsPerLoad / kDmaWaves;   // per issuing wave
  static constexpr int kBLoads = BNW / kRowsPerLoad / kDmaWaves;
  static constexpr int kDmaPerWave = kALoads + kBLoads;
  static_assert(WM * WN == kWaves && NT >= 1 && MT >= 1, "wave grid");
  static_assert(kAStages >= 2 && kAStages <= 3 && kBStages >= 2 && kBStages <= 4, "rings");
  static_assert(kLdsBytes <= 160 * 1024, "LDS of one CU");
  // load i of every issuing wave reads the same operand: 0 activations, 1 the first weight
  // operand (gate with SwiGLU), 2 the up weights
  static_assert((BM / kRowsPerLoad) % kDmaWaves == 0 &&
                    (BNW / 2 / kRowsPerLoad) % kDmaWaves == 0,
                "direct loads per wave: each load index stays within one operand");
  template <bool SWIGLU>
  __device__ static constexpr int kind_of(int i) {
    return i < kALoads ? 0 : !SWIGLU || (i - kALoads) * kDmaWaves * kRowsPerLoad < BNW / 2 ? 1 : 2;
  }
  // slot of k-chunk c in row r: c ^ swz(r); conflict-free 32x32 fragment reads (measured)
  __device__ static inline int swz(int r) {
    return ROWB == 64 ? ((r >> 2) & 3) : ((r >> 1) & 7);
  }
};
// The tile P as it runs on element type T (M16_ = 2 resolved to the 16x16 form for bf16).
template <class P, class T>
struct ForElt {
  using type = P;
};
template <int R, int S, int BM, int BNW, int WM, int WN, int D, int BS, class T>
struct ForElt<PrefillTileT<R, S, BM, BNW, WM, WN, D, BS, 2>, T> {
  using type = PrefillTileT<R, S, BM, BNW, WM, WN, D, BS, sizeof(T) == 2 ? 1 : 0>;
};

// Prefill: 256 x 256 tile, two 64 KB stages of 128-byte row pieces, 16x16 MFMA tiles.
using PrefillTile = PrefillTileT<128, 2, 256, 256, 2, 4, 1, 3, 1>;
// Prefill with tall experts: 320 x 256 tile, two 72 KB stages (142 flop per loaded byte).
using PrefillTallTile = PrefillTileT<128, 2, 320, 256, 2, 4, 1, 0, 2>;
// An expert's last row tile when it holds at most 128 rows: 128 x 256, the weight ring
// three deep (the same weight columns as the full tiles).
using PrefillTailTile = PrefillTileT<128, 2, 128, 256, 2, 4, 1, 3, 2>;
// ... and twice as wide (two n-tiles) for the last tile of an expert with at least two full
// 320-row tiles: 128 x 512, two 80 KB stages.
using PrefillTailWideTile = PrefillTileT<128, 2, 128, 512, 2, 4, 1, 2, 2>;
// Decode: weight streaming.  64 x 256 tile, three 40 KB stages, so two stages (80 KB per
// CU) of weight reads are in flight while one is multiplied.
using DecodeDmaTile = PrefillTileT<128, 3, 64, 256, 2, 4>;
// Router logits in dense mode: 64 tokens x 128 experts, one 32x32 tile per wave, so a
// DeepSeek-V3-sized router (8192 tokens, 256 experts) spreads over 256 blocks.
using RouterTile = PrefillTileT<128, 3, 64, 128, 2, 4>;
// Down GEMM of decode-sized experts: the same 64 x 128 tile.  Its short reduction (F) makes
// every tile start wait for a full HBM round trip; at 72 KB of LDS two blocks share a CU
// and one streams while the other starts (decode layer -1.5 % against 64 x 256).
using DecodeDownTile = PrefillTileT<128, 3, 64, 128, 2, 4>;

// A wave-uniform 64-bit address, moved to scalar registers.
__device__ inline uint64_t uniform_u64(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return ((uint64_t)hi << 32) | lo;
}
// Raw buffer resource for byte offsets below 2^31 from a uniform base address.  Selecting
// between bases (scalar) rather than between descriptors keeps the descriptor in scalar
// registers; a descriptor the compiler cannot prove uniform turns every buffer load into a
// serialised per-lane loop.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(uint64_t base) {
  constexpr int kFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(base), 0, 0x7fffffff,
                                           kFlags);
}

template <int N>
using IntC = std::integral_constant<int, N>;
// f(IntC<0>{}), ..., f(IntC<L-1>{}), with compile-time indices
template <class F, int... Is>
__device__ inline void unroll_steps_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(IntC<Is>{}), ...);
}
template <int L, class F>
__device__ inline void unroll_steps(F&& f) {
  unroll_steps_impl(f, std::make_integer_sequence<int, L>{});
}

// wait until at most N direct loads of this wave are outstanding, then block barrier
template <int N>
__device__ inline void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <class T, bool SWIGLU, class P, class OutT, int kLdsAlloc>
__device__ __attribute__((always_inline)) inline void prefill_gemm_body(
    const T* __restrict__ A, const int32_t* __restrict__ a_rows, const T* __restrict__ B0,
    const T* __restrict__ B1, int64_t b_expert_stride, OutT* __restrict__ C,
    const float* __restrict__ col_bias, float* __restrict__ Cacc, int K, int N_out, int e,
    int m_begin, int m_end, int nt, int k_first, int k_steps, bool stream_b,
    lds_char* __restrict__ a0, lds_char* __restrict__ a1,
    lds_char* __restrict__ a2, lds_char* __restrict__ b0, lds_char* __restrict__ b1,
    lds_char* __restrict__ b2, lds_char* __restrict__ b3) {
  constexpr int BN = SWIGLU ? P::BNW / 2 : P::BNW;
  static_assert(!SWIGLU || P::NT % 2 == 0, "SwiGLU pairs gate and up tiles in each wave");

  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int wm = wave / P::WN, wn = wave % P::WN;
  const int64_t row_bytes = (int64_t)K * sizeof(T);

  // Direct loads.  A stage of the activation ring holds the BM activation rows; a stage of
  // the weight ring the weight rows, with SwiGLU the BNW/2 gate rows first and the BNW/2
  // up rows of the same output columns after them.  Each load fills one block of
  // kRowsPerLoad rows; load i of issuing wave `dslot` fills block i * kDmaWaves + dslot of
  // the concatenated rows (activations, then weights), so the operand a load reads
  // (kind_of(i)) is the same for every issuing wave and known at compile time.  Each
  // operand is addressed through a buffer resource based at the tile's first row: a lane's
  // source is a 32-bit offset (row within the tile, clamped to the valid rows, times the row
  // pitch, plus its swizzled chunk) and the stage's k offset is a scalar.  Clamped rows are
  // loaded but their results never stored.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool issuer = P::kDmaSel == 0 || wave_u >= 4;
  const int dslot = P::kDmaSel == 0 ? wave_u : wave_u - 4;
  const T* B0e = B0 + (int64_t)e * b_expert_stride;
  const T* B1e = SWIGLU ? B1 + (int64_t)e * b_expert_stride : nullptr;
  // activation rows: rows m_begin.. of A, or (gathered) the A rows a_rows[m_begin..]
  const uint64_t base[3] = {uniform_u64(a_rows ? A : A + (int64_t)m_begin * K),
                            uniform_u64(B0e + (int64_t)nt * BN * K),
                            SWIGLU ? uniform_u64(B1e + (int64_t)nt * BN * K) : 0};
  constexpr int kBRows = SWIGLU ? P::BNW / 2 : P::BNW;  // rows of one weight operand
  uint32_t voff[P::kDmaPerWave];
#pragma unroll
  for (int i = 0; i < P::kDmaPerWave; ++i) {
    const int kind = P::template kind_of<SWIGLU>(i);
    // row of the lane within its ring's stage buffer
    const int r = ((kind == 0 ? i : i - P::kALoads) * P::kDmaWaves + dslot) * P::kRowsPerLoad +
                  lane / P::kChunks;
    const int c = (lane % P::kChunks) ^ P::swz(r);
    int row = kind == 0 ? min(r, m_end - 1 - m_begin)
                        : min(r - (kind - 1) * kBRows, N_out - 1 - nt * BN);
    if (kind == 0 && a_rows) {  // an empty padded slot (-1) reads row 0; never stored
      const int src = a_rows[m_begin + row];
      row = src < 0 ? 0 : src;
    }
    voff[i] = (uint32_t)row * (uint32_t)row_bytes + (uint32_t)(c * 16);
  }
  const int dma_lds = dslot * 1024;

  // accumulators of the wave's 32x32 tiles: one f32x16 each, or (M16) 2 x 2 f32x4 of the
  // 16x16 tiles [activation half][output-column half]
  using AccT = typename std::conditional<P::kM16, f32x4[2][2], f32x16>::type;
  AccT acc[P::MT][P::NT];
#pragma unroll
  for (int i = 0; i < P::MT; ++i)
#pragma unroll
    for (int j = 0; j < P::NT; ++j) {
      if constexpr (P::kM16) {
#pragma unroll
        for (int h = 0; h < 4; ++h) acc[i][j][h / 2][h % 2] = f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
      }
    }

  // a wave whose band of MT x 32 rows lies past the expert's rows skips its MFMAs; in a
  // band that ends inside the expert's last rows, the 32-row tiles past them (mt_live and
  // on) skip theirs (the band's waves run the partial copy of the multiply, see step)
  const bool band_live = m_begin + wm * P::MT * 32 < m_end;
  const int mt_live = __builtin_amdgcn_readfirstlane(
      band_live ? min(P::MT, (m_end - m_begin - wm * P::MT * 32 + 31) / 32) : 0);
  // lane l supplies row l % FR of an operand fragment and its k-chunk l / FR of the k-step
  constexpr int FR = P::kFragRows, SUB = P::kSub;
  const int frag_row = lane & (FR - 1), frag_k = lane / FR;
  const int a_frag = (wm * P::MT * 32 + frag_row) * P::kRowBytes;
  // weight rows of this wave: NT tiles of 32; with SwiGLU NT/2 gate tiles (from the gate
  // half of the stage) and the NT/2 up tiles of the same output columns
  constexpr int kNG = SWIGLU ? P::NT / 2 : P::NT;
  const int b_frag = (wn * kNG * 32 + frag_row) * P::kRowBytes;
  const int swz = P::swz(frag_row);

  // stages k_first .. k_first + k_steps - 1 of the reduction (all of it, or one piece)
  const int KT = k_steps;
  constexpr int SA = P::kAStages, SB = P::kBStages;
  constexpr int DA = SA - 1, DB = SB - 1;  // stages of each ring in flight ahead
  constexpr int nA = P::kALoads, nB = P::kBLoads;
  // Loads a wave may leave outstanding at the top of step k, when stage k of both rings must
  // have landed: each step issues its activation loads, then its weight loads, and with
  // DA < DB the activation stage k is the later of the two to be issued.
  constexpr int kWait = DA == DB ? (DA - 1) * (nA + nB)
                        : DA < DB ? nB + (DA - 1) * (nA + nB)
                                  : (DB - 1) * (nA + nB);
  // Stage buffers by compile-time index (indices fold to the distinct pointers).
  auto ring_a = [&](auto I) -> lds_char* {
    constexpr int j = decltype(I)::value % SA;
    return j == 0 ? a0 : j == 1 ? a1 : a2;
  };
  auto ring_b = [&](auto I) -> lds_char* {
    constexpr int j = decltype(I)::value % SB;
    return j == 0 ? b0 : j == 1 ? b1 : j == 2 ? b2 : b3;
  };
  // Direct load i of stage kt into its ring's buffer.  Stages past the end re-read the last
  // stage (k offset clamped, always in bounds) into a buffer nobody reads again, so every
  // step issues the same number of loads and the wait count is a constant.
  // With stream_b the weight loads carry the non-temporal hint: the plan sets it when each
  // weight line is read by about one tile, and then it keeps the streamed weights from
  // displacing the activation rows the other tiles reuse.
  // With two stages in each ring every step waits for all of a wave's loads (kWait = 0),
  // so the number of loads may vary: an activation load whose rows all lie past the
  // expert's last row is skipped (its LDS rows feed only outputs that are never stored).
  // A step is bound by the loads' issue and latency, so the partial tiles get cheaper.
  // (bf16 only: the test would cost the fp32 instances registers)
  constexpr bool kSkipDeadRows = SA == 2 && SB == 2 && sizeof(T) == 2;
  const int m_rows = m_end - m_begin;
  auto dma = [&](int i, int kt, lds_char* buf) {
    const uint32_t koff = (uint32_t)(k_first + min(kt, KT - 1)) * P::kRowBytes;
    const int blk = (i < nA ? i : i - nA) * P::kDmaWaves;
    if (kSkipDeadRows && i < nA && (blk + dslot) * P::kRowsPerLoad >= m_rows) return;
    const auto rsrc = buffer_rsrc(base[P::template kind_of<SWIGLU>(i)]);
    if (i >= nA && stream_b)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, buf + dma_lds + blk * 1024, 16, voff[i],
                                               koff, 0, 2 /* non-temporal */);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, buf + dma_lds + blk * 1024, 16, voff[i],
                                               koff, 0, 0);
  };
  auto dma_a = [&](int kt, lds_char* buf) {
    if (!issuer) return;
#pragma unroll
    for (int i = 0; i < nA; ++i) dma(i, kt, buf);
  };
  auto dma_b = [&](int kt, lds_char* buf) {
    if (!issuer) return;
#pragma unroll
    for (int i = nA; i < nA + nB; ++i) dma(i, kt, buf);
  };
  // Fragments of one k-step: SUB per 32 rows of the MT activation tiles and the NT weight
  // tiles (fragment SUB * t + h holds rows t * 32 + FR * h ..).
  auto load_frags = [&](const lds_char* abuf, const lds_char* bbuf, int ks, u32x4* fa,
                        u32x4* fb) {
    const int slot = ((ks * P::kStepChunks + frag_k) ^ swz) << 4;
#pragma unroll
    for (int j = 0; j < P::NT; ++j)
#pragma unroll
      for (int h = 0; h < SUB; ++h)
        fb[SUB * j + h] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            bbuf + b_frag + ((j < kNG ? 0 : kBRows - kNG * 32) + j * 32 + FR * h) *
                                P::kRowBytes + slot);
#pragma unroll
    for (int i = 0; i < P::MT; ++i)
#pragma unroll
      for (int h = 0; h < SUB; ++h)
        fa[SUB * i + h] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            abuf + a_frag + (i * 32 + FR * h) * P::kRowBytes + slot);
  };
  // Multiply one stage.  The reads of k-step s+1 go out between the MFMAs of k-step s (two
  // register sets), so each k-step's MFMAs cover the next k-step's LDS latency.
  // live: the 32-row tiles of the band that hold rows (compile-time; step picks the copy)
  auto compute = [&](const lds_char* abuf, const lds_char* bbuf, auto live) {
    constexpr int LIVE = decltype(live)::value;
    if (!band_live) return;
    u32x4 fa[2][SUB * P::MT], fb[2][SUB * P::NT];
    load_frags(abuf, bbuf, 0, fa[0], fb[0]);
#pragma unroll
    for (int ks = 0; ks < P::kKSteps; ++ks) {
      if (ks + 1 < P::kKSteps)
        load_frags(abuf, bbuf, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < P::MT; ++i) {
        if (i >= LIVE) continue;
#pragma unroll
        for (int hi = 0; hi < SUB; ++hi)
#pragma unroll
          for (int j = 0; j < P::NT; ++j)
#pragma unroll
            for (int hj = 0; hj < SUB; ++hj) {
              if constexpr (P::kM16)
                mma_chunk(acc[i][j][hi][hj], fb[ks & 1][2 * j + hj], fa[ks & 1][2 * i + hi],
                          T());
              else
                mma32_chunk(acc[i][j], fb[ks & 1][j], fa[ks & 1][i], T());
            }
      }
      // order: [reads of step 0]; per step, its MFMAs with the next step's reads spread
      // evenly between them (read r goes before MFMA floor(r * M / R)); measured about 1 %
      // faster on the prefill layers than issuing the reads as one burst
      if (ks == 0) __builtin_amdgcn_sched_group_barrier(0x100, SUB * (P::MT + P::NT), 0);
      if (ks + 1 < P::kKSteps) {
        constexpr int R = SUB * (P::MT + P::NT), M = SUB * SUB * P::MT * P::NT;
        unroll_steps<M>([&](auto MI) {
          constexpr int m = decltype(MI)::value;
          constexpr int r_lo = (m * R + M - 1) / M, r_hi = ((m + 1) * R + M - 1) / M;
          if constexpr (r_hi > r_lo) __builtin_amdgcn_sched_group_barrier(0x100, r_hi - r_lo, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        });
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, SUB * SUB * P::MT * P::NT, 0);
      }
    }
  };
  // The 16x16 form with many activation tiles per wave (P::kLean): the double-buffered
  // schedule above would hold 2 x (2 MT + 2 NT) fragments and spill the 320-row tile.  Here
  // the weight fragments of a k-step are double-buffered across k-steps, while the
  // activation fragments stream through a ring of three items (an item = the two 16-row
  // fragments of one 32-row tile), each loaded two items (16 MFMAs of this wave) before its
  // MFMAs: 2 NT + 3 SUB fragments instead of 2 (2 MT + 2 NT).  Same products in the same
  // order per accumulator as compute().
  auto compute_lean = [&](const lds_char* abuf, const lds_char* bbuf, auto live) {
    if constexpr (P::kLean) {
    constexpr int LIVE = decltype(live)::value;
    if (!band_live) return;
    constexpr int KS = P::kKSteps, NI = KS * P::MT, RING = 3;
    u32x4 fb[2][SUB * P::NT], fa[RING][SUB];
    auto ld_b = [&](int ks, u32x4* dst) {
      const int slot = ((ks * P::kStepChunks + frag_k) ^ swz) << 4;
#pragma unroll
      for (int j = 0; j < P::NT; ++j)
#pragma unroll
        for (int h = 0; h < SUB; ++h)
          dst[SUB * j + h] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
              bbuf + b_frag + ((j < kNG ? 0 : kBRows - kNG * 32) + j * 32 + FR * h) *
                                  P::kRowBytes + slot);
    };
    auto ld_a = [&](int ks, int i, u32x4* dst) {
      const int slot = ((ks * P::kStepChunks + frag_k) ^ swz) << 4;
#pragma unroll
      for (int h = 0; h < SUB; ++h)
        dst[h] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            abuf + a_frag + (i * 32 + FR * h) * P::kRowBytes + slot);
    };
    ld_b(0, fb[0]);
    unroll_steps<RING - 1>([&](auto N) {
      constexpr int n = decltype(N)::value;
      ld_a(n / P::MT, n % P::MT, fa[n]);
    });
    __builtin_amdgcn_sched_group_barrier(0x100, SUB * P::NT + (RING - 1) * SUB, 0);
    unroll_steps<NI>([&](auto N) {
      constexpr int n = decltype(N)::value, ks = n / P::MT, i = n % P::MT;
      constexpr int nl = n + RING - 1;  // the item whose fragments are loaded now
      constexpr bool load_a = nl < NI;
      constexpr bool load_b = i == 1 && ks + 1 < KS;  // the next k-step's weight fragments
      if constexpr (load_a) ld_a(nl / P::MT, nl % P::MT, fa[nl % RING]);
      if constexpr (load_b) ld_b(ks + 1, fb[(ks + 1) & 1]);
      if constexpr (i < LIVE) {
#pragma unroll
        for (int hi = 0; hi < SUB; ++hi)
#pragma unroll
          for (int j = 0; j < P::NT; ++j)
#pragma unroll
            for (int hj = 0; hj < SUB; ++hj)
              mma_chunk(acc[i][j][hi][hj], fb[ks & 1][SUB * j + hj], fa[n % RING][hi], T());
      }
      // this item's loads first, then its MFMAs, the loads spread between them
      constexpr int R = (load_a ? SUB : 0) + (load_b ? SUB * P::NT : 0);
      constexpr int M = SUB * SUB * P::NT;
      unroll_steps<M>([&](auto MI) {
        constexpr int m = decltype(MI)::value;
        constexpr int r_lo = (m * R + M - 1) / M, r_hi = ((m + 1) * R + M - 1) / M;
        if constexpr (r_hi > r_lo) __builtin_amdgcn_sched_group_barrier(0x100, r_hi - r_lo, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      });
    });
    }
  };
  // Step kt (I = kt modulo the unroll): wait until stage kt of both rings has landed, make
  // every wave's loads visible, issue activation stage kt + DA and weight stage kt + DB into
  // the buffers step kt-1 finished reading, then multiply.  The loads of a step go out
  // together after the barrier (spreading them between the MFMAs measured no faster).
  // The issuing wave of each SIMD multiplies only after it has issued its stage's loads, so
  // its MFMAs end the step; it takes precedence over its partner wave (measured 0.3-0.6 %
  // faster on the prefill layers, the reverse order 0.8 % slower).
  if (P::kDmaSel == 1 && issuer) __builtin_amdgcn_s_setprio(3);
  auto step = [&](int kt, auto I, auto live) {
    if (kt >= KT) return;
    wait_vm_barrier<kWait>();
    dma_a(kt + DA, ring_a(IntC<decltype(I)::value + DA>{}));
    dma_b(kt + DB, ring_b(IntC<decltype(I)::value + DB>{}));
    if constexpr (P::kLean)
      compute_lean(ring_a(I), ring_b(I), live);
    else
      compute(ring_a(I), ring_b(I), live);
  };

  // prologue: the loads of steps -max(DA, DB) .. -1, issued as those steps would
  constexpr int DM = DA > DB ? DA : DB;
  unroll_steps<DM>([&](auto V) {
    constexpr int v = decltype(V)::value - DM;
    if constexpr (v + DA >= 0) dma_a(v + DA, ring_a(IntC<v + DA>{}));
    if constexpr (v + DB >= 0) dma_b(v + DB, ring_b(IntC<v + DB>{}));
  });
  constexpr int L = SA == SB ? SA : SB % SA == 0 ? SB : SA * SB;  // the rings repeat
  // one copy of the k-loop per count of live 32-row tiles, so that no multiply tests tiles
  // inside its MFMA stream (the wave's count is the same for every step)
  auto k_loop = [&](auto live) {
    for (int kt = 0; kt < KT; kt += L) unroll_steps<L>([&](auto I) {
      step(kt + decltype(I)::value, I, live);
    });
  };
  // (bf16 only: the fp32 tiles keep one copy, which fits their registers)
  if (sizeof(T) != 2 || mt_live == P::MT || mt_live == 0) {
    k_loop(IntC<P::MT>{});
  } else {
    unroll_steps<P::MT - 1>([&](auto V) {
      constexpr int v = decltype(V)::value + 1;
      if (mt_live == v) k_loop(IntC<v>{});
    });
  }
  // drain the loads issued past the last stage before the block's LDS can be reassigned
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Epilogue.  The weight fragment is the MFMA's first operand, so each accumulator tile
  // is the transposed product: lane L holds activation row L % 32 of the 32 and, in
  // acc[.][.][4a + b], output column 8a + 4 (L / 32) + b; with 16x16 tiles, activation row
  // 16 hi + L % 16 and, in acc[.][.][hi][a][b], output column 16a + 4 (L / 16) + b.  The
  // block's outputs go through LDS in row-major order (4 consecutive columns per lane
  // write) and leave it as 16-byte stores that cover whole cache lines; storing one element
  // per lane per instruction straight from the accumulators took 7-17 % of a tile's time
  // (measured per block).
  // A piece of a split reduction stores its fp32 partial sums the same way.
  __syncthreads();  // every wave's direct loads have landed and its fragment reads are done
  constexpr int NOUT = SWIGLU ? P::NT / 2 : P::NT;
  const int q4 = 4 * frag_k;
  auto acc_at = [&](int i, int j, int hi, int a, int b) -> float {
    if constexpr (P::kM16)
      return acc[i][j][hi][a][b];
    else
      return acc[i][j][4 * a + b];
  };
  auto staged = [&](auto st_tag, auto rd_tag, auto emit) {
    using ST = decltype(st_tag);                       // staged element type
    constexpr int RD = decltype(rd_tag)::value;        // bytes each lane reads back
    constexpr int kRow = BN * (int)sizeof(ST);         // bytes of one staged row
    constexpr int kChunks = kRow / 16;
    static_assert(kChunks >= 16 && kChunks % 16 == 0, "swizzle spans 16 chunks");
    constexpr int kTileRows = P::WM * 32;              // one row tile of every wave band
    constexpr int IP0 = kLdsAlloc / (kTileRows * kRow);
    constexpr int IP = IP0 < P::MT ? IP0 : P::MT;      // row tiles per pass
    static_assert(IP >= 1, "one row tile of the output fits the block's LDS");
    constexpr int kPer = kTileRows * IP * kRow / RD;   // lane reads per pass
#pragma unroll
    for (int p0 = 0; p0 < P::MT; p0 += IP) {
      if (p0 > 0) __syncthreads();  // the previous pass has been read back
      if (band_live) {
#pragma unroll
        for (int ii = 0; ii < IP; ++ii) {
          const int i = p0 + ii;
          if (i >= P::MT) break;
#pragma unroll
          for (int hi = 0; hi < SUB; ++hi) {
          const int srow = (wm * IP + ii) * 32 + FR * hi + frag_row;
          lds_char* rowp = a0 + srow * kRow;
#pragma unroll
          for (int j = 0; j < NOUT; ++j)
#pragma unroll
            for (int a = 0; a < 4 / SUB; ++a) {
              const int cb = (((wn * NOUT + j) * 32 + 8 * SUB * a + q4) * (int)sizeof(ST));
              const int off = (((cb >> 4) ^ (srow & 15)) << 4) | (cb & 15);
              float v[4];
#pragma unroll
              for (int b = 0; b < 4; ++b)
                v[b] = SWIGLU ? silu_f32(acc_at(i, j, hi, a, b)) * acc_at(i, j + NOUT, hi, a, b)
                              : acc_at(i, j, hi, a, b);
              if constexpr (sizeof(ST) == 4) {
                *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(rowp + off) =
                    f32x4{v[0], v[1], v[2], v[3]};
              } else {
                typedef ST stx4 __attribute__((ext_vector_type(4)));
                *reinterpret_cast<__attribute__((address_space(3))) stx4*>(rowp + off) =
                    stx4{Elt<ST>::from_f32(v[0]), Elt<ST>::from_f32(v[1]),
                         Elt<ST>::from_f32(v[2]), Elt<ST>::from_f32(v[3])};
              }
            }
          }
        }
      }
      __syncthreads();
#pragma unroll 2
      for (int it = 0; it < (kPer + P::kThreads - 1) / P::kThreads; ++it) {
        const int q = it * P::kThreads + tid;
        if (kPer % P::kThreads != 0 && q >= kPer) break;
        const int srow = q / (kRow / RD), cbyte = (q % (kRow / RD)) * RD;
        const int band = srow / (IP * 32), ii = (srow / 32) % IP;
        const int row = m_begin + band * P::MT * 32 + (p0 + ii) * 32 + (srow & 31);
        const int col = nt * BN + cbyte / (int)sizeof(ST);
        if (p0 + ii >= P::MT || row >= m_end || col >= N_out) continue;
        const int off = (((cbyte >> 4) ^ (srow & 15)) << 4) | (cbyte & 15);
        emit(row, col, a0 + srow * kRow + off);
      }
    }
  };
  if (!SWIGLU && Cacc) {  // one piece of a split reduction: its tile of fp32 partial sums
    staged(float(), IntC<16>{}, [&](int row, int col, const lds_char* src) {
      *reinterpret_cast<f32x4*>(Cacc + (int64_t)(row - m_begin) * BN + (col - nt * BN)) =
          *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(src);
    });
  } else if constexpr (std::is_same<OutT, float>::value) {  // fp32 output
    staged(float(), IntC<16>{}, [&](int row, int col, const lds_char* src) {
      f32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(src);
      float* dst = C + (int64_t)row * N_out + col;
      if (col_bias)
#pragma unroll
        for (int b = 0; b < 4; ++b) v[b] += col_bias[min(col + b, N_out - 1)];
      if (N_out % 4 == 0) {
        *reinterpret_cast<f32x4*>(dst) = v;
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (col + b < N_out) dst[b] = v[b];
      }
    });
  } else {  // bf16 output: N_out is a multiple of 128, so every chunk is whole and aligned
    staged(OutT(), IntC<16>{}, [&](int row, int col, const lds_char* src) {
      *reinterpret_cast<u32x4*>(C + (int64_t)row * N_out + col) =
          *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(src);
    });
  }
}

// Stage buffers of tile P in the block's LDS, then its body.
template <class T, bool SWIGLU, class P, class OutT, int kLdsAlloc>
__device__ __attribute__((always_inline)) inline void prefill_gemm_tile(
    const T* __restrict__ A, const int32_t* __restrict__ a_rows, const T* __restrict__ B0,
    const T* __restrict__ B1, int64_t b_expert_stride, OutT* __restrict__ C,
    const float* __restrict__ col_bias, float* __restrict__ Cacc, int K, int N_out, int e,
    int m_begin, int m_end, int nt, int k_first, int k_steps, bool stream_b, lds_char* base) {
  constexpr int SA = P::kABytes, SB = P::kBBytes;
  lds_char* bb = base + P::kAStages * SA;
  // buffers past a ring's stage count are never used
  prefill_gemm_body<T, SWIGLU, typename ForElt<P, T>::type, OutT, kLdsAlloc>(
      A, a_rows, B0, B1, b_expert_stride, C, col_bias, Cacc, K, N_out, e, m_begin, m_end, nt,
      k_first, k_steps, stream_b, base, base + SA, base + (P::kAStages > 2 ? 2 * SA : 0), bb,
      bb + SB, bb + (P::kBStages > 2 ? 2 * SB : 0), bb + (P::kBStages > 3 ? 3 * SB : 0));
}

// Down GEMM with few, long tiles: the tail split.  The t = m-tiles x n-tiles tiles (m-tiles
// counted on the device) are numbered densely, n fastest within groups of group_n n-tiles.
// The first floor(t / cus) * cus tiles run whole; the tail of t mod cus tiles, which would
// leave most CUs idle through a last partial round, is split along the reduction into
// S = min(s_max, cus / tail) pieces, each storing its tile of fp32 partial sums in a slot of
// its own for tail_sum_kernel to add in piece order (deterministic).  S < 2: nothing splits.
struct TailSplit {
  int tiles, whole, tail, pieces;
};
__device__ inline TailSplit tail_split_of(int m_tiles, int n_tiles, int s_max) {
  TailSplit p;
  p.tiles = m_tiles * n_tiles;
  p.whole = p.tiles / kSplitCUs * kSplitCUs;
  p.tail = p.tiles - p.whole;
  p.pieces = p.tail ? min(s_max, kSplitCUs / p.tail) : 1;
  if (p.pieces < 2) {
    p.whole = p.tiles;
    p.tail = 0;
    p.pieces = 1;
  }
  return p;
}
// (m-tile, n-tile) of dense tile number i: groups of m_tiles x group_n tiles, n fastest
// within a group; the last group holds the n_tiles mod group_n remaining n-tiles.
__device__ inline void dense_tile(int i, int m_tiles, int n_tiles, int group_n, int* mt,
                                  int* nt) {
  const int per_group = m_tiles * group_n, full = n_tiles / group_n;
  if (i < full * per_group) {
    const int grp = i / per_group, rem = i - grp * per_group;
    *mt = rem / group_n;
    *nt = grp * group_n + rem % group_n;
  } else {
    const int rem = i - full * per_group, gw = n_tiles - full * group_n;
    *mt = rem / gw;
    *nt = full * group_n + rem % gw;
  }
}

// One block per (m-tile, n-tile), or, with the tail split, per whole tile or per piece of a
// tail tile.  Blocks are dealt round-robin to the 8 XCDs; the logical tile index is
// remapped so each XCD walks a contiguous range of logical tiles, n fastest within
// groups of group_n n-tiles (with the tail split: XCD x runs its share of the whole tiles
// first, so the first round holds whole tiles only, then its share of the pieces).
// An m-tile with at most PT::BM rows (an expert's last, partly
// filled tile) runs the shorter tile PT with the same weight columns: fewer loads and MFMAs
// instead of a full tile of mostly clamped rows.  When PW is twice as wide as P, the last
// tile of an expert with at least two full tiles runs PW over n-tiles nt and nt + 1 in the
// block of the even nt (the odd one exits): a short tile of single width runs about twice
// as fast as the full tiles beside it and races ahead through the weight panel they share
// in L2, so they miss; the double-width one keeps their pace.  Measured with the 320-row
// tile: Mixtral-8x7B layer -2.8 %; experts with fewer full tiles keep PT, since with one
// full tile (Mixtral-8x22B) the pairing's halved block count costs more than it saves.
// When PM is shorter than P and taller than PT, an m-tile of PT::BM + 1 ... PM::BM rows (an
// expert's last tile) runs PM: the 320-row gate/up GEMM gives such tiles the 256-row tile,
// whose deeper weight ring hides more of the load latency that bounds a partly filled
// tall tile (Mixtral-8x22B gate/up -2 %; its down GEMM gained nothing and keeps P).
//
// Dense mode (table == nullptr, used for the router logits): one operand A of dense_rows
// rows and one B of N_out rows, m-tile mt covering rows mt * P::BM ...
template <class T, bool SWIGLU, class P, class PT, class OutT, class PW, class PM>
__global__ void __launch_bounds__(P::kThreads)
prefill_gemm_kernel(const T* __restrict__ A, const int32_t* __restrict__ a_rows,
                    const T* __restrict__ B0, const T* __restrict__ B1,
                    int64_t b_expert_stride, OutT* __restrict__ C,
                    const float* __restrict__ col_bias, float* __restrict__ Cacc, int K,
                    int N_out, const int32_t* __restrict__ offsets,
                    const int32_t* __restrict__ table, int m_tiles_max, int n_tiles,
                    int group_n, int grid_logical, int tail_split, int dense_rows,
                    int stream_b) {
  static_assert(PT::BNW == P::BNW && PT::kThreads == P::kThreads && PT::BM <= P::BM,
                "the shorter tile shares the n-tiling and the block size");
  static_assert((PW::BNW == P::BNW || PW::BNW == 2 * P::BNW) && PW::BM == PT::BM &&
                    PW::kThreads == P::kThreads,
                "the wide tail tile spans one or two n-tiles of the full tile");
  static_assert(PM::BNW == P::BNW && PM::kThreads == P::kThreads && PM::BM <= P::BM,
                "the medium tile shares the n-tiling and the block size");
  extern __shared__ __attribute__((aligned(1024))) char smem_dyn[];
  // dynamic LDS of the launch (launch_prefill allocates the largest of the three tiles)
  constexpr int kLds =
      std::max({P::kLdsBytes, PT::kLdsBytes, PW::kLdsBytes, PM::kLdsBytes});
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int per_xcd = gridDim.x >> 3;
  // stages [k_first, k_first + k_steps) of the reduction: all of it, or one piece of a tail
  // tile, whose fp32 partial sums go to its slot of Cacc
  const int KT = K * (int)sizeof(T) / P::kRowBytes;
  int mt, nt, k_first = 0, k_steps = KT;
  float* acc = nullptr;
  if (tail_split > 0) {  // tile-table mode only (launch_prefill refuses other uses)
    const int m_tiles = table[0];
    const TailSplit ts = tail_split_of(m_tiles, n_tiles, tail_split);
    const int w8 = (ts.whole + 7) / 8, q8 = (ts.tail * ts.pieces + 7) / 8;
    int tile;
    if (j < w8) {
      tile = xcd * w8 + j;
      if (tile >= ts.whole) return;
    } else {
      const int q = xcd * q8 + (j - w8);
      if (j - w8 >= q8 || q >= ts.tail * ts.pieces) return;
      const int piece = q / ts.tail;
      tile = ts.whole + (q - piece * ts.tail);
      k_first = piece * KT / ts.pieces;
      k_steps = (piece + 1) * KT / ts.pieces - k_first;
      acc = Cacc + ((int64_t)(tile - ts.whole) * ts.pieces + piece) * (P::BM * P::BNW);
    }
    dense_tile(tile, m_tiles, n_tiles, group_n, &mt, &nt);
  } else {
    const int logical = xcd * per_xcd + j;
    if (logical >= grid_logical) return;
    const int per_group = m_tiles_max * group_n;
    const int grp = logical / per_group, rem = logical - grp * per_group;
    mt = rem / group_n;
    nt = grp * group_n + (rem - (rem / group_n) * group_n);
    if (nt >= n_tiles) return;
  }
  int e, m_begin, m_end;
  if (table) {
    if (mt >= table[0]) return;
    e = table[1 + 2 * mt];
    m_begin = table[2 + 2 * mt];
    m_end = offsets[e + 1];
  } else {
    e = 0;
    m_begin = mt * P::BM;
    m_end = min(dense_rows, m_begin + P::BM);
    if (m_begin >= m_end) return;
  }
  lds_char* base = (lds_char*)smem_dyn;
  if constexpr (PM::BM < P::BM && PM::BM > PT::BM) {
    if (table && m_end - m_begin > PT::BM && m_end - m_begin <= PM::BM) {
      prefill_gemm_tile<T, SWIGLU, PM, OutT, kLds>(A, a_rows, B0, B1, b_expert_stride, C,
                                                   col_bias, acc, K, N_out, e, m_begin, m_end,
                                                   nt, k_first, k_steps, stream_b != 0, base);
      return;
    }
  }
  if (PT::BM < P::BM && m_end - m_begin <= PT::BM) {
    if constexpr (PW::BNW == 2 * P::BNW) {
      // at least two full tiles before (not with the tail split, whose pieces each hold
      // the partial sums of one n-tile)
      if (table && tail_split == 0 && m_begin - offsets[e] >= 2 * P::BM) {
        if (nt & 1) return;
        prefill_gemm_tile<T, SWIGLU, PW, OutT, kLds>(A, a_rows, B0, B1, b_expert_stride, C,
                                               col_bias, acc, K, N_out, e, m_begin, m_end,
                                               nt >> 1, k_first, k_steps,
                                               stream_b != 0, base);
        return;
      }
    }
    prefill_gemm_tile<T, SWIGLU, PT, OutT, kLds>(A, a_rows, B0, B1, b_expert_stride, C, col_bias,
                                           acc, K, N_out, e, m_begin, m_end, nt,
                                           k_first, k_steps, stream_b != 0, base);
  } else
    prefill_gemm_tile<T, SWIGLU, P, OutT, kLds>(A, a_rows, B0, B1, b_expert_stride, C,
                                                col_bias, acc, K, N_out, e, m_begin, m_end,
                                                nt, k_first, k_steps, stream_b != 0, base);
}

// The tail tiles of a tail-split down GEMM: tile i (dense number whole + i) is the sum of
// its S slots of fp32 partial sums ([BM, BN] each, slot i * S + p), added in piece order so
// the result does not depend on which piece finished first, converted to the output type
// and stored into the tile's valid rows and columns.  grid = (kSplitCUs, any): blockIdx.x
// is the tail tile (surplus blocks exit), blockIdx.y strides over its float4 groups.
template <class T, int BM, int BN>
__global__ void __launch_bounds__(256)
tail_sum_kernel(const float* __restrict__ acc, const int32_t* __restrict__ offsets,
                const int32_t* __restrict__ table, int n_tiles, int group_n, int s_max,
                int N_out, T* __restrict__ y) {
  const int m_tiles = table[0];
  const TailSplit ts = tail_split_of(m_tiles, n_tiles, s_max);
  const int i = blockIdx.x;
  if (i >= ts.tail) return;
  int mt, nt;
  dense_tile(ts.whole + i, m_tiles, n_tiles, group_n, &mt, &nt);
  const int e = table[1 + 2 * mt], m_begin = table[2 + 2 * mt];
  const int rows = min(offsets[e + 1] - m_begin, BM), cols = min(BN, N_out - nt * BN);
  const float* src = acc + (int64_t)i * ts.pieces * (BM * BN);
  for (int f = blockIdx.y * 256 + threadIdx.x; f < rows * (BN / 4); f += gridDim.y * 256) {
    const int r = f / (BN / 4), c = (f % (BN / 4)) * 4;
    if (c >= cols) continue;
    f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + r * BN + c));
    for (int p = 1; p < ts.pieces; ++p) {
      const f32x4 w = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(src + (int64_t)p * (BM * BN) + r * BN + c));
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] += w[q];
    }
    T* dst = y + (int64_t)(m_begin + r) * N_out + nt * BN + c;
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = Elt<T>::from_f32(v[q]);
  }
}

// ---------------------------------------------------------------------------------------
// launch configurations
// ---------------------------------------------------------------------------------------
// Row-tile heights: decode-sized experts (mean <= 32 rows) stream weights with 64-row tiles;
// prefill-sized ones use 256- or 320-row tiles.
FfnPlan ffn_plan(int64_t T, int64_t E, int64_t k, int64_t C, int64_t R, bool pad, int64_t d,
                 int64_t F, int64_t elt) {
  FfnPlan p;
  p.small = pad ? C <= 32 : T * k <= 32 * E;
  if (p.small) {
    p.tile = 0;
    p.bm = DecodeDmaTile::BM;
    p.stream_b = true;  // a few rows per expert: every weight line is read by one tile
    p.group_cap = 4;
  } else {
    // Rows an expert will probably hold: a little above the mean, at most the capacity.
    // Take the tile height that needs fewer row tiles (each one re-reads the expert's
    // weight panel), then the one that pads fewer rows.
    const int64_t mean = (T * k + E - 1) / E;
    int64_t r = pad ? C : mean + mean / 20;
    if (r > C) r = C;
    const int64_t t256 = (r + 255) / 256, t320 = (r + 319) / 320;
    const bool tall = t320 < t256 || (t320 == t256 && t320 * 320 < t256 * 256);
    p.tile = tall ? 2 : 1;
    p.bm = tall ? PrefillTallTile::BM : PrefillTile::BM;
    // An expert's weight panel is re-read by each of its row tiles, through L2 while they
    // run together.  With at most two row tiles per expert the weights are effectively
    // streamed and take the non-temporal hint (measured: DeepSeek-V3 mixed batch -4 %,
    // Mixtral-8x22B -3.5 %); with four (Mixtral-8x7B) the hint costs 7 %.
    p.stream_b = (r + p.bm - 1) / p.bm <= 2;
    // Launch order: each XCD walks groups of (all m-tiles) x group_cap n-tiles.  When an
    // expert fits one row tile and its weights stream, the activation rows are the only
    // operand reused, so a group spans every n-tile (DeepSeek-V3 mixed batch -3 %);
    // otherwise 8 n-tiles, which lets an expert's row tiles share its weight panel.
    p.group_cap = p.stream_b && r <= p.bm ? (1 << 30) : 8;
  }
  int64_t m_max = (R + E * (p.bm - 1)) / p.bm;
  const int64_t m_cap = E * ((C + p.bm - 1) / p.bm);
  p.m_max = m_cap < m_max ? m_cap : m_max;
  if (p.m_max < 0) p.m_max = 0;
  // Down GEMM with few, long tiles: when the tile count (at most m_max x ceil(d / 256))
  // is below two rounds of the 256 CUs, the last, partial round would leave most of the
  // chip idle for a whole tile time.  The GEMM then runs the tail split (tail_split_of):
  // the tiles of the last partial round, counted on the device, are split along the
  // reduction into up to down_split pieces (at most 8, at least 16 128-byte stages each)
  // whose fp32 partial sums another launch adds in piece order.  Only those tiles pay for
  // partial sums (at most 256 pieces of BM x 256 floats); the whole tiles store their
  // outputs directly.  This replaced a split of every tile into three pieces on the
  // Mixtral-8x22B layer (288 tiles: 256 whole, 32 in eight pieces).
  p.down_split = 1;
  p.down_pieces_max = 0;
  const int64_t tiles = p.m_max * ((d + 255) / 256), stages = F * elt / 128;
  if (!p.small && tiles > 0 && tiles < 2 * kSplitCUs) {
    const int64_t split = std::min<int64_t>(8, stages / 16);
    if (split >= 2) {
      p.down_split = (int)split;
      p.down_pieces_max = std::min<int64_t>(kSplitCUs, tiles * split);
    }
  }
  return p;
}

// Upper bound on the blocks of either grouped-GEMM launch of plan p (launch_prefill): at
// most m_max x (n-tiles rounded up to whole groups, < 2 x n-tiles) logical tiles of at least
// 128 columns, rounded up to a multiple of 8, plus the tail split's pieces.
int64_t ffn_max_blocks(const FfnPlan& p, int64_t d, int64_t F) {
  const int64_t n128 = ((d > F ? d : F) + 127) / 128;
  return p.m_max * 2 * n128 + 8 + kSplitCUs;
}

namespace {

// tail_split > 0 (tile-table mode, no SwiGLU): the tail split with at most tail_split pieces
// per tail tile, partial sums in c_acc, then tail_sum_kernel.
template <class T, bool SW, class P = PrefillTile, class PT = PrefillTailTile, class OutT = T,
          class PW = PT, class PM = P>
hipError_t launch_prefill(const T* A, const int32_t* a_rows, const T* B0, const T* B1,
                          int64_t b_stride, OutT* C, int K, int N_out, const int32_t* offsets,
                          const int32_t* table, int64_t m_max, hipStream_t s, int tail_split,
                          float* c_acc, const float* col_bias, int dense_rows, bool stream_b,
                          int group_cap) {
  if (m_max <= 0) return hipSuccess;
  // the tail split runs over a tile table, without SwiGLU, into a partial-sum buffer
  if (tail_split > 0 && (SW || !table || !c_acc || !std::is_same<OutT, T>::value))
    return hipErrorInvalidValue;
  constexpr int BN = SW ? P::BNW / 2 : P::BNW;
  const int n_tiles = (N_out + BN - 1) / BN;
  const int group_n = n_tiles < group_cap ? n_tiles : group_cap;
  const int n_groups = (n_tiles + group_n - 1) / group_n;
  const int64_t logical = m_max * group_n * n_groups;
  // with the tail split, each XCD's share of the whole tiles (at most m_max x n_tiles of
  // them) and of the pieces (at most kSplitCUs)
  const int64_t grid = tail_split > 0 ? 8 * ((m_max * n_tiles + 7) / 8 + kSplitCUs / 8)
                                      : (logical + 7) / 8 * 8;
  const size_t lds =
      (size_t)std::max({P::kLdsBytes, PT::kLdsBytes, PW::kLdsBytes, PM::kLdsBytes});
  hipError_t e = hipFuncSetAttribute((const void*)prefill_gemm_kernel<T, SW, P, PT, OutT, PW, PM>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  prefill_gemm_kernel<T, SW, P, PT, OutT, PW, PM><<<(unsigned)grid, P::kThreads, lds, s>>>(
      A, a_rows, B0, B1, b_stride, C, col_bias, c_acc, K, N_out, offsets, table, (int)m_max,
      n_tiles, group_n, (int)logical, tail_split, dense_rows, stream_b ? 1 : 0);
  if ((e = hipGetLastError()) != hipSuccess || tail_split == 0) return e;
  if constexpr (!SW && std::is_same<OutT, T>::value) {
    tail_sum_kernel<T, P::BM, P::BNW><<<dim3(kSplitCUs, 8), 256, 0, s>>>(
        c_acc, offsets, table, n_tiles, group_n, tail_split, N_out, C);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

hipError_t launch_table(const FfnArgs& a, const FfnPlan& p, hipStream_t s) {
  if (p.m_max <= 0) return hipSuccess;
  tile_table_kernel<<<1, 1024, 0, s>>>(a.offsets, (int)a.E, p.bm, (int)p.m_max, a.sched);
  return hipGetLastError();
}

template <class T>
hipError_t run_gate_up(const FfnArgs& a, const FfnPlan& p, hipStream_t s) {
  // activations: x_perm, or x with the rows gathered through a.src_rows
  const T* xp = (const T*)(a.src_rows ? a.x : a.x_perm);
  const int32_t* rows = a.src_rows;
  T* h = (T*)a.h;
  const int64_t stride = a.F * a.d;
  const T* wg = (const T*)a.w_gate;
  const T* wu = (const T*)a.w_up;
  // no tail split (0), no partial sums, no column bias, tile-table mode (0 dense rows)
  if (p.small)
    return launch_prefill<T, true, DecodeDmaTile, DecodeDmaTile>(
        xp, rows, wg, wu, stride, h, (int)a.d, (int)a.F, a.offsets, a.sched, p.m_max, s, 0,
        nullptr, nullptr, 0, p.stream_b, p.group_cap);
  if (p.tile == 2)
    return launch_prefill<T, true, PrefillTallTile, PrefillTailTile, T, PrefillTailWideTile,
                          PrefillTile>(
        xp, rows, wg, wu, stride, h, (int)a.d, (int)a.F, a.offsets, a.sched, p.m_max, s, 0,
        nullptr, nullptr, 0, p.stream_b, p.group_cap);
  return launch_prefill<T, true>(xp, rows, wg, wu, stride, h, (int)a.d, (int)a.F, a.offsets,
                                 a.sched, p.m_max, s, 0, nullptr, nullptr, 0, p.stream_b,
                                 p.group_cap);
}

template <class T>
hipError_t run_down(const FfnArgs& a, const FfnPlan& p, hipStream_t s) {
  const T* h = (const T*)a.h;
  T* y = (T*)a.y_perm;
  const int64_t stride = a.d * a.F;
  if (p.small)
    return launch_prefill<T, false, DecodeDownTile, DecodeDownTile>(
        h, nullptr, (const T*)a.w_down, nullptr, stride, y, (int)a.F, (int)a.d, a.offsets,
        a.sched, p.m_max, s, 0, nullptr, nullptr, 0, p.stream_b, p.group_cap);
  // tail split: the tiles of the last partial round run in pieces (see ffn_plan)
  const int ts = p.down_split > 1 ? p.down_split : 0;
  float* acc = ts ? a.down_acc : nullptr;
  if (p.tile == 2)
    return launch_prefill<T, false, PrefillTallTile, PrefillTailTile, T, PrefillTailWideTile>(
        h, nullptr, (const T*)a.w_down, nullptr, stride, y, (int)a.F, (int)a.d, a.offsets,
        a.sched, p.m_max, s, ts, acc, nullptr, 0, p.stream_b, p.group_cap);
  return launch_prefill<T, false>(h, nullptr, (const T*)a.w_down, nullptr, stride, y, (int)a.F,
                                  (int)a.d, a.offsets, a.sched, p.m_max, s, ts, acc, nullptr, 0,
                                  p.stream_b, p.group_cap);
}

}  // namespace

// Router logits L = x w^T (+ b) through the same pipeline in dense mode: 64-token x
// 128-expert tiles, fp32 output with the bias added in the epilogue.  Used when there are
// enough tiles to spread over the CUs.
// (At most 2^22 tiles, so the launch stays within 2^31 threads; larger shapes take the
// router kernel, whose blocks stride over the token tiles.)
bool router_gemm_suits(int64_t T, int64_t E) {
  const int64_t tiles = ((T + RouterTile::BM - 1) / RouterTile::BM) *
                        ((E + RouterTile::BNW - 1) / RouterTile::BNW);
  return E >= 64 && tiles >= 192 && tiles <= ((int64_t)1 << 22);
}

hipError_t launch_router_gemm(int dtype, const void* x, const void* w, const float* b,
                              float* logits, int64_t T, int64_t d, int64_t E, hipStream_t s) {
  const int64_t m_tiles = (T + RouterTile::BM - 1) / RouterTile::BM;
  // dense mode: no tile table, no tail split, the bias in the epilogue, n-groups of 8
  if (dtype == 1)
    return launch_prefill<bf16, false, RouterTile, RouterTile, float>(
        (const bf16*)x, nullptr, (const bf16*)w, nullptr, 0, logits, (int)d, (int)E, nullptr,
        nullptr, m_tiles, s, 0, nullptr, b, (int)T, false, 8);
  return launch_prefill<float, false, RouterTile, RouterTile, float>(
      (const float*)x, nullptr, (const float*)w, nullptr, 0, logits, (int)d, (int)E, nullptr,
      nullptr, m_tiles, s, 0, nullptr, b, (int)T, false, 8);
}

hipError_t launch_expert_ffn(const FfnArgs& a, int which, hipStream_t s) {
  if (a.R <= 0) return hipSuccess;
  const FfnPlan p = ffn_plan(a.T, a.E, a.k, a.C, a.R, a.pad, a.d, a.F, a.dtype == 1 ? 2 : 4);
  if (p.down_split > 1 && (which & 2) && !a.down_acc) return hipErrorInvalidValue;
  hipError_t err = a.table_ready ? hipSuccess : launch_table(a, p, s);
  if (err != hipSuccess) return err;
  if (which & 1) {
    err = a.dtype == 1 ? run_gate_up<bf16>(a, p, s) : run_gate_up<float>(a, p, s);
    if (err != hipSuccess) return err;
  }
  if (which & 2) err = a.dtype == 1 ? run_down<bf16>(a, p, s) : run_down<float>(a, p, s);
  return err;
}

}  // namespace moe
