// Internal building blocks of the MoE kernels for gfx950 (CDNA4): 16-byte memory chunks,
// the 16x16 (router) and 32x32 (expert GEMM) MFMA tiles, bf16 conversion and wave scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------------------
// element traits: one 16-byte chunk holds kPerChunk elements
// ---------------------------------------------------------------------------------------
template <class T>
struct Elt;
template <>
struct Elt<float> {
  static constexpr int kPerChunk = 4;
  __device__ static inline float to_f32(float v) { return v; }
  __device__ static inline float from_f32(float v) { return v; }
};
template <>
struct Elt<bf16> {
  static constexpr int kPerChunk = 8;
  __device__ static inline float to_f32(bf16 v) { return (float)v; }
  __device__ static inline bf16 from_f32(float v) { return (bf16)v; }  // round to nearest even
};

__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// ---------------------------------------------------------------------------------------
// 16x16 output tile, one 16-byte chunk of A and of B per lane per call.
//
// Lane l supplies row (l % 16) of A and row (l % 16) of B (B is stored [n][k], i.e. the
// GEMM is C = A B^T with both operands contiguous along k) and the chunk at k-chunk
// position (l / 16) of the current 64-byte k-step.  The result tile holds
// C[4 * (l / 16) + i][l % 16] in acc[i].
//   bf16: one v_mfma_f32_16x16x32_bf16 (8 elements per lane per chunk).
//   fp32: four v_mfma_f32_16x16x4_f32, element i of the chunk in the i-th one.  Each
//         k-position is covered exactly once for A and B alike, so the sum is the same.
// ---------------------------------------------------------------------------------------
__device__ inline void mma_chunk(f32x4& acc, const u32x4& a, const u32x4& b, bf16) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ inline void mma_chunk(f32x4& acc, const u32x4& a, const u32x4& b, float) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[i]), __uint_as_float(b[i]),
                                               acc, 0, 0, 0);
}

// ---------------------------------------------------------------------------------------
// 32x32 output tile, one 16-byte chunk of A and of B per lane per call.
//
// Lane l supplies row (l % 32) of A and of B (B stored [n][k]) and the chunk at k-chunk
// position (l / 32) of the current 32-byte k-step.  The result tile holds
// C[8 * (i / 4) + 4 * (l / 32) + (i % 4)][l % 32] in acc[i], i < 16.
//   bf16: one v_mfma_f32_32x32x16_bf16.  On gfx950 both this instruction and the 16x16x32
//         form sustain the full dense bf16 rate per clock (2.48 PFLOP/s over the chip on
//         zero operands); on random data the 16x16x32 form holds a higher clock under the
//         power limit (1.94 against 1.75 GHz in a register-only loop), so the prefill tiles
//         use that form and this one serves the HBM-bound decode tiles, where the 32x32
//         tile's fragments take half the registers.
//   fp32: four v_mfma_f32_32x32x2_f32, element i of the chunk in the i-th one.
// ---------------------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ inline void mma32_chunk(f32x16& acc, const u32x4& a, const u32x4& b, bf16) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ inline void mma32_chunk(f32x16& acc, const u32x4& a, const u32x4& b, float) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i]), __uint_as_float(b[i]),
                                               acc, 0, 0, 0);
}

// ---------------------------------------------------------------------------------------
// wave helpers
// ---------------------------------------------------------------------------------------
__device__ inline int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ inline uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m, kWave);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// Inclusive prefix sum over a wave.
__device__ inline int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

// Exclusive prefix sum of one value per thread over a block of up to 1024 threads
// (blockDim.x a multiple of 64).  `smem` needs 17 ints.  Returns the exclusive prefix;
// *total gets the block sum.  Contains barriers: every thread of the block must call it.
__device__ inline int block_exclusive_scan(int v, int* smem, int* total) {
  const int lane = lane_id(), wave = threadIdx.x / kWave, nwaves = blockDim.x / kWave;
  int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) smem[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int w = lane < nwaves ? smem[lane] : 0;
    int wi = wave_inclusive_scan(w);
    if (lane < nwaves) smem[lane] = wi - w;
    if (lane == kWave - 1) smem[16] = wi;
  }
  __syncthreads();
  int res = smem[wave] + inc - v;
  *total = smem[16];
  __syncthreads();
  return res;
}

}  // namespace moe
