// S8: gate-weighted combine back to token order.
//
// [EP-serving] aiunderstanding.org, "Expert parallelism for MoE serving", section
// "Technical details": the combine step brings expert outputs back to their tokens.  On one
// GPU it is a gather: every token reads its k expert rows through dest_row (the inverse of
// the dispatch permutation), so no two threads write the same output and no atomics are
// needed.  Slots are summed in order 0..k-1 in fp32, which makes the result deterministic.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

// Token t, column segment seg: lane l sums 16-byte chunk seg * 64 + l of the token's
// expert rows.
template <class T, int G>
__device__ inline void combine_item(const T* __restrict__ y, const int32_t* __restrict__ dest,
                                    const float* __restrict__ w, T* __restrict__ out, int d,
                                    int k, int64_t t, int seg) {
  constexpr int P = Elt<T>::kPerChunk;
  const int c = seg * kWave + lane_id();  // 16-byte chunk of the row
  if (c >= d / P) return;
  const int32_t* dt = dest + t * k;
  const float* wt = w + t * k;
  float acc[P];
#pragma unroll
  for (int i = 0; i < P; ++i) acc[i] = 0.f;
  // slots in groups of G: the group's row loads go out together, the sums still run in
  // slot order
  for (int j0 = 0; j0 < k; j0 += G) {
    u32x4 v[G];
    float g[G];
    bool live[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int j = j0 + u;
      const int r = j < k ? dt[j] : -1;
      live[u] = r >= 0;
      g[u] = live[u] ? wt[j] : 0.f;
      v[u] = live[u] ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                           y + (int64_t)r * d + (int64_t)c * P))
                     : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (!live[u]) continue;  // dropped slots add nothing
      const T* e = reinterpret_cast<const T*>(&v[u]);
#pragma unroll
      for (int i = 0; i < P; ++i) acc[i] = fmaf(g[u], Elt<T>::to_f32(e[i]), acc[i]);
    }
  }
  u32x4 o;
  T* oe = reinterpret_cast<T*>(&o);
#pragma unroll
  for (int i = 0; i < P; ++i) oe[i] = Elt<T>::from_f32(acc[i]);
  // y_perm rows are read once and out written once: streaming (non-temporal) accesses
  // keep them from displacing other lines in the caches (15 % faster at k = 8, d = 7168)
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + t * d + (int64_t)c * P));
}

// One wave per (token, 64-chunk column segment): lane l of segment s sums chunk
// s * 64 + l of the token's k expert rows.  Splitting each row over several waves keeps
// enough loads in flight when T is small (a decode step of 256 tokens x 14 segments).
// The grid is capped (launch_combine) and the waves stride over the T * segs work items,
// so any T * d fits the launch limits.
template <class T, int G>
__global__ void __launch_bounds__(256)
combine_kernel(const T* __restrict__ y, const int32_t* __restrict__ dest,
               const float* __restrict__ w, T* __restrict__ out, int64_t T_, int d, int k,
               int segs) {
  const int wave = threadIdx.x / kWave;
  const int64_t items = T_ * segs;
  for (int64_t gw = (int64_t)blockIdx.x * 4 + wave; gw < items; gw += (int64_t)gridDim.x * 4)
    combine_item<T, G>(y, dest, w, out, d, k, gw / segs, (int)(gw % segs));
}

hipError_t launch_combine(int dtype, const void* y_perm, const int32_t* dest_row,
                          const float* topk_w, void* out, int64_t T, int64_t d, int64_t k,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int per_chunk = dtype == 1 ? 8 : 4;
  const int segs = (int)((d / per_chunk + kWave - 1) / kWave);
  // at most 2^20 blocks (4 waves each); the waves stride over the rest
  const unsigned blocks = (unsigned)std::min<int64_t>((T * segs + 3) / 4, 1 << 20);
  // slot groups of 8 when k is large enough to fill them, else 4
  if (dtype == 1 && k > 4)
    combine_kernel<bf16, 8><<<blocks, 256, 0, s>>>((const bf16*)y_perm, dest_row, topk_w,
                                                   (bf16*)out, T, (int)d, (int)k, segs);
  else if (dtype == 1)
    combine_kernel<bf16, 4><<<blocks, 256, 0, s>>>((const bf16*)y_perm, dest_row, topk_w,
                                                   (bf16*)out, T, (int)d, (int)k, segs);
  else if (k > 4)
    combine_kernel<float, 8><<<blocks, 256, 0, s>>>((const float*)y_perm, dest_row, topk_w,
                                                    (float*)out, T, (int)d, (int)k, segs);
  else
    combine_kernel<float, 4><<<blocks, 256, 0, s>>>((const float*)y_perm, dest_row, topk_w,
                                                    (float*)out, T, (int)d, (int)k, segs);
  return hipGetLastError();
}

}  // namespace moe
