// S1 router logits and S2 top-k gating.
//
// [EP-serving] aiunderstanding.org, "Expert parallelism for MoE serving", section "Deep
// dive": a router chooses the top-k experts of every token.  The layer specification fixes
// the rest: fp32 logits, softmax top-k with ties to the lower expert index, and gates
// renormalised over the selection.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------------------
// small utility: zero an int32 buffer (used instead of a memset node so that the sequence
// stays capturable in a HIP graph)
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) zero_i32_kernel(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  zero_i32_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// S1: L[t, e] = sum_i x[t, i] w[e, i] + b[e]
//
// The router GEMM is skinny (E = 8 or 256 columns) and bound by reading x (and, for
// E = 256, w) once.  A block computes a (16 * MT)-token x (16 * NT)-expert tile with MFMA
// straight from global memory (no LDS staging); its W waves split the reduction axis in
// 128-byte steps (wave w takes steps w, w + W, ...), each wave loading its next step while
// multiplying the current one, and their partial tiles are summed in LDS in wave order,
// which keeps the result deterministic.  Per 128-byte step a lane loads 32 contiguous bytes
// of each of its MT token rows and NT expert rows; both operands use the same k-chunk
// assignment (lane group g takes chunks 2g and 2g + 1), so the products pair up.  Each load
// touches half of 16 cache lines, so shapes with many tokens and experts (enough 64 x 128
// tiles to fill the CUs) go through the expert-GEMM pipeline instead.
// grid = (min(ceil(T / (16 MT)), 2^16), ceil(E / (16 NT))): the blocks of a column of the
// grid stride over the token tiles.  With status_zero set, the first thread of block (0, 0)
// also clears that word (the top-k kernel after this one counts into it), which saves the
// layer a launch.
// ---------------------------------------------------------------------------------------
template <class T, int MT, int NT, int kRouterWaves>
__device__ __attribute__((always_inline)) inline void router_logits_tile(
    const T* __restrict__ x, const T* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ logits, int T_, int d, int E, int t0, int e0, float* part) {
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const char* xa[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int t = min(t0 + m * 16 + r, T_ - 1);  // clamped rows are computed, never stored
    xa[m] = reinterpret_cast<const char*>(x + (int64_t)t * d) + g * 32;
  }
  const char* wb[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int e = min(e0 + n * 16 + r, E - 1);
    wb[n] = reinterpret_cast<const char*>(w + (int64_t)e * d) + g * 32;
  }
  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int steps = d * (int)sizeof(T) / 128;
  // operands of one 128-byte step; the next step's loads go out before this step's MFMAs
  u32x4 a0[2][MT], a1[2][MT], b0[2][NT], b1[2][NT];
  auto load = [&](int st, int set) {
    const int kb = st * 128;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      a0[set][m] = ld16(xa[m] + kb);
      a1[set][m] = ld16(xa[m] + kb + 16);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      b0[set][n] = ld16(wb[n] + kb);
      b1[set][n] = ld16(wb[n] + kb + 16);
    }
  };
  auto mfma = [&](int set) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        mma_chunk(acc[m][n], a0[set][m], b0[set][n], T());
        mma_chunk(acc[m][n], a1[set][m], b1[set][n], T());
      }
  };
  if (wave < steps) load(wave, 0);
  for (int st = wave; st < steps; st += 2 * kRouterWaves) {
    if (st + kRouterWaves < steps) load(st + kRouterWaves, 1);
    mfma(0);
    if (st + kRouterWaves >= steps) break;
    if (st + 2 * kRouterWaves < steps) load(st + 2 * kRouterWaves, 0);
    mfma(1);
  }
  constexpr int kTile = MT * NT * 4 * kWave;  // floats of one wave's partial tile
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        part[wave * kTile + ((m * NT + n) * 4 + i) * kWave + lane] = acc[m][n][i];
  __syncthreads();
  // thread -> (m, n, i, lane) of the tile; sum the W partial tiles in wave order
  for (int o = threadIdx.x; o < kTile; o += blockDim.x) {
    const int mn = o / (4 * kWave), i = (o / kWave) % 4, l = o % kWave;
    const int m = mn / NT, n = mn % NT;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < kRouterWaves; ++ww) v += part[ww * kTile + o];
    const int e = e0 + n * 16 + (l & 15);
    const int tt = t0 + m * 16 + 4 * (l >> 4) + i;
    if (e < E && tt < T_) logits[(int64_t)tt * E + e] = v + (bias ? bias[e] : 0.f);
  }
}

template <class T, int MT, int NT, int kRouterWaves>
__global__ void __launch_bounds__(kRouterWaves* kWave)
router_logits_kernel(const T* __restrict__ x, const T* __restrict__ w,
                     const float* __restrict__ bias, float* __restrict__ logits, int T_,
                     int d, int E, int32_t* __restrict__ status_zero) {
  extern __shared__ float part[];  // [W][MT][NT][4][kWave]
  if (status_zero && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *status_zero = 0;
  const int tiles = (T_ + MT * 16 - 1) / (MT * 16);
  for (int tb = blockIdx.x; tb < tiles; tb += gridDim.x) {
    router_logits_tile<T, MT, NT, kRouterWaves>(x, w, bias, logits, T_, d, E, tb * MT * 16,
                                                blockIdx.y * NT * 16, part);
    __syncthreads();  // the partial tiles have been read before the next tile writes them
  }
}

template <class T, int MT, int NT, int W>
hipError_t launch_router_tile(const T* x, const T* w, const float* b, float* logits,
                              int64_t T_, int64_t d, int64_t E, int32_t* status_zero,
                              hipStream_t s) {
  const size_t lds = (size_t)W * MT * NT * 4 * kWave * sizeof(float);
  hipError_t e = hipFuncSetAttribute((const void*)router_logits_kernel<T, MT, NT, W>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)std::min<int64_t>((T_ + 16 * MT - 1) / (16 * MT), 1 << 16),
                  (unsigned)((E + 16 * NT - 1) / (16 * NT)));
  router_logits_kernel<T, MT, NT, W><<<grid, W * kWave, lds, s>>>(x, w, b, logits, (int)T_,
                                                                  (int)d, (int)E, status_zero);
  return hipGetLastError();
}

template <class T>
hipError_t launch_router_typed(const T* x, const T* w, const float* b, float* logits,
                               int64_t T_, int64_t d, int64_t E, int32_t* status_zero,
                               hipStream_t s) {
  // 16 x 64 tiles when that still gives at least 512 blocks (two per CU), else 16 x 16
  // (larger shapes take the GEMM pipeline, see launch_router_logits).  With at most 512
  // blocks of 16 x 16 (a decode step, or E = 8 with up to 8192 tokens) each CU holds one or
  // two blocks, whose loads are all the CU has in flight: 16 waves split the reduction then.
  const int64_t t16 = (T_ + 15) / 16;
  if (E > 16 && t16 * ((E + 63) / 64) >= 512)
    return launch_router_tile<T, 1, 4, 8>(x, w, b, logits, T_, d, E, status_zero, s);
  if (t16 * ((E + 15) / 16) <= 512)
    return launch_router_tile<T, 1, 1, 16>(x, w, b, logits, T_, d, E, status_zero, s);
  return launch_router_tile<T, 1, 1, 8>(x, w, b, logits, T_, d, E, status_zero, s);
}

hipError_t launch_router_logits(int dtype, const void* x, const void* w, const float* b,
                                float* logits, int64_t T, int64_t d, int64_t E,
                                int32_t* status_zero, hipStream_t s) {
  if (T == 0) return status_zero ? launch_zero_i32(status_zero, 1, s) : hipSuccess;
  // many tokens and experts: full-line direct loads into LDS and 32x32 MFMA tiles (the
  // expert-GEMM pipeline); the kernel below reads half cache lines per load
  if (router_gemm_suits(T, E)) {
    hipError_t e = status_zero ? launch_zero_i32(status_zero, 1, s) : hipSuccess;
    return e != hipSuccess ? e : launch_router_gemm(dtype, x, w, b, logits, T, d, E, s);
  }
  if (dtype == 1)
    return launch_router_typed<bf16>((const bf16*)x, (const bf16*)w, b, logits, T, d, E,
                                     status_zero, s);
  return launch_router_typed<float>((const float*)x, (const float*)w, b, logits, T, d, E,
                                    status_zero, s);
}

// ---------------------------------------------------------------------------------------
// S2: top-k under (value descending, index ascending) and renormalised gates.
//
// A group of G lanes (G = power of two >= min(E, 64)) handles one token; lane s of the
// group holds experts s, s + G, s + 2G, ... as 64-bit keys
//     key = ordered(value) << 32 | (0xFFFFFFFF - e),
// where ordered() maps fp32 to an unsigned integer of the same order (after turning -0.0
// into +0.0).  Larger key = better expert; equal values compare by the low word, which
// prefers the lower index.  k rounds of a group max-reduction pick the experts in order.
// Non-finite logits are counted into *status (one per token) and get key 0 (every finite
// logit's key is non-zero, its low word alone being at least 0xFFFFFC00).
//
// The selection value is the logit, or the fp32 sum logit + sel_bias[e] when a
// selection-only bias is given; the gates always use the logits.
//
// Group-limited selection (NG > 1 groups of E / NG consecutive experts, keep M groups): a
// group's key is the largest key of its experts (its best value; equal values favour the
// lower expert index and so the lower group).  NG rounds of a group reduction leave group
// g's key on lane g (NG <= G); M rounds of a max-reduction over those pick the groups, and
// the keys of experts outside them are cleared before the k rounds.
// ---------------------------------------------------------------------------------------
template <int N>
using IntC32 = std::integral_constant<int, N>;

__device__ inline uint32_t ordered_f32(float v) {
  if (v == 0.0f) v = 0.0f;  // -0.0 == +0.0
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// max of v over the G lanes of this lane group (G a power of two <= 64)
__device__ inline uint64_t group_max_u64(uint64_t v, int G) {
  for (int msk = G >> 1; msk > 0; msk >>= 1) {
    const uint64_t o = shfl_xor_u64(v, msk);
    v = o > v ? o : v;
  }
  return v;
}
__device__ inline float group_max_f32(float v, int G) {
  for (int msk = G >> 1; msk > 0; msk >>= 1) v = fmaxf(v, __shfl_xor(v, msk, kWave));
  return v;
}
__device__ inline float group_sum_f32(float v, int G) {
  for (int msk = G >> 1; msk > 0; msk >>= 1) v += __shfl_xor(v, msk, kWave);
  return v;
}

template <int V>
__global__ void __launch_bounds__(256)
topk_kernel(const float* __restrict__ logits, const float* __restrict__ sel_bias,
            int64_t T_, int E, int k, int G, int NG, int M, int32_t* __restrict__ topk_idx,
            float* __restrict__ topk_w, int32_t* __restrict__ status) {
  // Grid-stride over groups of G lanes in 64-bit indices (T * G may pass 2^31).  G divides
  // the wave, so a wave's tokens lie in one pass and the loop condition is wave-uniform:
  // every lane of a wave runs the same passes, as the group shuffles below require.
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t wave0 = (int64_t)blockIdx.x * blockDim.x + (threadIdx.x & ~(kWave - 1));
       wave0 / G < T_; wave0 += stride) {
    const int64_t gtid = wave0 + lane_id();
    const int64_t tok = gtid / G;
    const int sub = (int)(gtid % G);
    const bool active = tok < T_;
    const float* row = logits + (active ? tok : 0) * E;

    uint64_t key[V];
    float lg[V];  // the logits of this lane's experts (the gates use them)
    int bad = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = sub + v * G;
      key[v] = 0;
      lg[v] = 0.f;
      if (active && e < E) {
        const float val = row[e];
        lg[v] = val;
        const float sv = sel_bias ? val + sel_bias[e] : val;
        if (__builtin_isfinite(val) && __builtin_isfinite(sv))
          key[v] = ((uint64_t)ordered_f32(sv) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
        else
          bad = 1;
      }
    }
    // group OR of the non-finite flag
    for (int m = G >> 1; m > 0; m >>= 1) bad |= __shfl_xor(bad, m, kWave);
    if (active && sub == 0 && bad && status) atomicAdd(status, 1);

    if (NG > 1 && M < NG) {
      const int gs = E / NG;
      uint64_t gkey = 0;  // lane g: key of group g
      for (int g = 0; g < NG; ++g) {
        uint64_t b = 0;
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const int e = sub + v * G;
          if (e < E && e / gs == g && key[v] > b) b = key[v];
        }
        b = group_max_u64(b, G);
        if (sub == g) gkey = b;
      }
      uint64_t chosen = 0;  // bit g: group g kept
      for (int r = 0; r < M; ++r) {
        const uint64_t b = group_max_u64(gkey, G);
        if (b == 0) break;  // only tokens with non-finite logits get here
        const int g = (int)(0xFFFFFFFFu - (uint32_t)b) / gs;
        chosen |= 1ull << g;
        if (sub == g) gkey = 0;
      }
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int e = sub + v * G;
        if (e < E && !((chosen >> (e / gs)) & 1ull)) key[v] = 0;
      }
    }

    // Slot 0 holds the best selection.  Round j's winner is expert e, held by lane e % G of
    // the group as its entry e / G; that lane's logit reaches the group by one shuffle and
    // lane j keeps slot j (k <= G).  The gates are exp(L_j - m) / sum with m the largest
    // selected logit, computed by the k slot lanes together.
    const int base = lane_id() & ~(G - 1);
    int slot_e = 0;
    float slot_l = -__builtin_huge_valf();
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int v = 0; v < V; ++v) best = key[v] > best ? key[v] : best;
      best = group_max_u64(best, G);
      // the unique owner retires the winning key
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (key[v] == best) key[v] = 0;
      const int e = best ? (int)(0xFFFFFFFFu - (uint32_t)best) : 0;
      float mine = 0.f;  // this lane's logit of expert e's column
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (v == e / G) mine = lg[v];
      const float l = __shfl(mine, base + e % G, kWave);
      if (sub == j) {
        slot_e = e;
        slot_l = l;
      }
    }
    const float m = group_max_f32(sub < k ? slot_l : -__builtin_huge_valf(), G);
    const float ex = sub < k ? expf(slot_l - m) : 0.f;
    const float inv = 1.0f / group_sum_f32(ex, G);
    if (active && sub < k) {
      topk_idx[tok * k + sub] = slot_e;
      topk_w[tok * k + sub] = ex * inv;
    }
  }
}

// The same selection for groups of at most 16 lanes (E <= 256 experts, k <= 16 slots,
// no group-limited selection): a group lies inside one 16-lane row of the wave, so its
// reductions are DPP moves (quad_perm [1,0,3,2] and [2,3,0,1], then row_half_mirror and
// row_mirror, which pair every lane with one lane of each larger block) instead of LDS
// permutes.  The k rounds only keep the winning expert on slot lane j; afterwards each slot
// lane reads its expert's logit back from the row the group has just read.  Same keys,
// same selection; the gates' sums run in another order (within the gate tolerance).
template <int CTRL>
__device__ inline uint32_t dpp_u32(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}
template <int CTRL>
__device__ inline float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
// op over the G lanes of a group (G a power of two <= 16, groups aligned to G lanes)
template <int G, class V, class Dpp, class Op>
__device__ inline V row_group_reduce(V v, Dpp dpp, Op op) {
  if constexpr (G > 1) v = op(v, dpp(v, IntC32<0xB1>{}));
  if constexpr (G > 2) v = op(v, dpp(v, IntC32<0x4E>{}));
  if constexpr (G > 4) v = op(v, dpp(v, IntC32<0x141>{}));
  if constexpr (G > 8) v = op(v, dpp(v, IntC32<0x140>{}));
  return v;
}

template <int G, int V>
__global__ void __launch_bounds__(256)
topk_row_kernel(const float* __restrict__ logits, const float* __restrict__ sel_bias,
                int64_t T_, int E, int k, int32_t* __restrict__ topk_idx,
                float* __restrict__ topk_w, int32_t* __restrict__ status) {
  auto d64 = [](uint64_t v, auto c) { return dpp_u64<decltype(c)::value>(v); };
  auto d32 = [](uint32_t v, auto c) { return dpp_u32<decltype(c)::value>(v); };
  auto df = [](float v, auto c) { return dpp_f32<decltype(c)::value>(v); };
  // grid-stride over the groups; G divides the wave, so the loop condition is wave-uniform
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t wave0 = (int64_t)blockIdx.x * blockDim.x + (threadIdx.x & ~(kWave - 1));
       wave0 / G < T_; wave0 += stride) {
    const int64_t gtid = wave0 + lane_id();
    const int64_t tok = gtid / G;
    const int sub = (int)(gtid % G);
    const bool active = tok < T_;
    const float* row = logits + (active ? tok : 0) * E;
    uint64_t key[V];
    uint32_t bad = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = sub + v * G;
      key[v] = 0;
      if (active && e < E) {
        const float val = row[e];
        const float sv = sel_bias ? val + sel_bias[e] : val;
        if (__builtin_isfinite(val) && __builtin_isfinite(sv))
          key[v] = ((uint64_t)ordered_f32(sv) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
        else
          bad = 1;
      }
    }
    bad = row_group_reduce<G>(bad, d32, [](uint32_t a, uint32_t b) { return a | b; });
    if (active && sub == 0 && bad && status) atomicAdd(status, 1);
    int slot_e = 0;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int v = 0; v < V; ++v) best = key[v] > best ? key[v] : best;
      best = row_group_reduce<G>(best, d64,
                                 [](uint64_t a, uint64_t b) { return a > b ? a : b; });
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (key[v] == best) key[v] = 0;  // the unique owner retires the winning key
      if (sub == j) slot_e = best ? (int)(0xFFFFFFFFu - (uint32_t)best) : 0;
    }
    const float slot_l = active && sub < k ? row[slot_e] : -__builtin_huge_valf();
    const float m = row_group_reduce<G>(slot_l, df, [](float a, float b) { return fmaxf(a, b); });
    const float ex = sub < k ? expf(slot_l - m) : 0.f;
    const float inv =
        1.0f / row_group_reduce<G>(ex, df, [](float a, float b) { return a + b; });
    if (active && sub < k) {
      topk_idx[tok * k + sub] = slot_e;
      topk_w[tok * k + sub] = ex * inv;
    }
  }
}

hipError_t launch_topk(const float* logits, const float* sel_bias, int64_t T, int64_t E,
                       int64_t k, int n_groups, int topk_groups, int32_t* idx, float* w,
                       int32_t* status, hipStream_t s) {
  if (T == 0) return hipSuccess;
  // groups inside a 16-lane row: DPP reductions
  if (!(n_groups > 1 && topk_groups < n_groups) && E <= 256 && k <= 16) {
    int G = 1;
    while (G < E && G < 16) G <<= 1;
    G = G < (int)k ? (int)k : G;  // k <= 16 slot lanes
    while (G & (G - 1)) ++G;      // (a power of two)
    const int V = (int)((E + G - 1) / G);
    const unsigned blocks = (unsigned)std::min<int64_t>((T * G + 255) / 256, 1 << 16);
#define MOE_TOPK_ROW(GG, VV)                                                             \
  topk_row_kernel<GG, VV><<<blocks, 256, 0, s>>>(logits, sel_bias, T, (int)E, (int)k,    \
                                                 idx, w, status)
    if (G == 1)
      MOE_TOPK_ROW(1, 1);
    else if (G == 2)
      MOE_TOPK_ROW(2, 1);
    else if (G == 4)
      MOE_TOPK_ROW(4, 1);
    else if (G == 8)
      MOE_TOPK_ROW(8, 1);
    else if (V <= 1)
      MOE_TOPK_ROW(16, 1);
    else if (V <= 2)
      MOE_TOPK_ROW(16, 2);
    else if (V <= 4)
      MOE_TOPK_ROW(16, 4);
    else if (V <= 8)
      MOE_TOPK_ROW(16, 8);
    else
      MOE_TOPK_ROW(16, 16);
#undef MOE_TOPK_ROW
    return hipGetLastError();
  }
  int G = 1;
  while (G < E && G < 64) G <<= 1;
  const int V = (int)((E + G - 1) / G);
  const int64_t threads = T * G;
  // at most 2^16 blocks; the kernel strides over the rest
  const unsigned blocks = (unsigned)std::min<int64_t>((threads + 255) / 256, 1 << 16);
#define MOE_TOPK(VV)                                                                     \
  topk_kernel<VV><<<blocks, 256, 0, s>>>(logits, sel_bias, T, (int)E, (int)k, G,         \
                                         n_groups, topk_groups, idx, w, status)
  if (V <= 1)
    MOE_TOPK(1);
  else if (V <= 2)
    MOE_TOPK(2);
  else if (V <= 4)
    MOE_TOPK(4);
  else if (V <= 8)
    MOE_TOPK(8);
  else
    MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace moe
