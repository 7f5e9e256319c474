// Calibration of the bf16 MFMA roofline on this GPU: the rate the chip sustains when every
// SIMD issues nothing but independent bf16 MFMAs (32x32x16, or 16x16x32 for comparison) on
// register operands, and the shader clock it holds meanwhile.  The published dense peak
// (2.5 PFLOP/s) assumes the full 2.4 GHz clock; under load the clock is set by the power
// limit, and the data the multipliers see moves it: random operands draw more power than
// zeros.  The GEMM kernels are measured
// against the published peak; this gives the ceiling beside it.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/moe_calib.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;       // two per SIMD, as in the GEMM kernels
constexpr int kChains = 4;      // independent accumulators per wave
constexpr int kLdsPad = 96 * 1024;  // keeps one block per CU (the LDS holds only one)

// 32-bit integer hash (the finaliser of MurmurHash3) of a counter.
__device__ inline uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x85ebca6bu;
  x ^= x >> 13;
  x *= 0xc2b2ae35u;
  x ^= x >> 16;
  return x;
}

// Two bf16 values with random sign and mantissa and magnitudes in [0.25, 4): operands with
// the bit statistics of normally distributed data.
__device__ inline uint32_t random_bf16_pair(uint32_t h) {
  const uint32_t lo = (h & 0x807fu) | ((125u + ((h >> 7) & 3u)) << 7);
  const uint32_t hi = ((h >> 16) & 0x807fu) | ((125u + ((h >> 23) & 3u)) << 7);
  return lo | (hi << 16);
}

// SHAPE 0: v_mfma_f32_32x32x16_bf16 (32768 flops, 16 accumulators per lane);
// SHAPE 1: v_mfma_f32_16x16x32_bf16 (16384 flops, 4 accumulators per lane).
template <int SHAPE>
__global__ __launch_bounds__(kWaves * 64) void mfma_rate_kernel(int iters, uint32_t seed,
                                                                int operands, float* sink,
                                                                unsigned long long* cycles) {
  typedef float accv __attribute__((ext_vector_type(SHAPE == 0 ? 16 : 4)));
  constexpr int kAcc = SHAPE == 0 ? 16 : 4;
  __shared__ float pad[kLdsPad / sizeof(float)];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u32x4 a[kChains], b[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t ctr = ((blockIdx.x * kWaves + wave) * 64 + lane) * (2 * kChains * 4) +
                           (j * 4 + q) * 2;
      a[j][q] = operands ? random_bf16_pair(hash32(ctr ^ seed)) : 0u;
      b[j][q] = operands ? random_bf16_pair(hash32((ctr + 1) ^ seed)) : 0u;
    }
  accv acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = accv{};
  __syncthreads();
  const unsigned long long c0 = clock64(), w0 = wall_clock64();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) {
      if constexpr (SHAPE == 0)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[j]),
                                                         __builtin_bit_cast(bf16x8, b[j]),
                                                         acc[j], 0, 0, 0);
      else
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[j]),
                                                         __builtin_bit_cast(bf16x8, b[j]),
                                                         acc[j], 0, 0, 0);
    }
  }
  const unsigned long long c1 = clock64(), w1 = wall_clock64();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int i = 0; i < kAcc; ++i) s += acc[j][i];
  // the LDS pad is touched only so the compiler keeps its allocation
  if (iters < 0) pad[threadIdx.x] = s;
  __syncthreads();
  if (iters < 0) s += pad[(threadIdx.x + 1) % (kWaves * 64)];
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) sink[blockIdx.x * kWaves + wave] = s;
  if (threadIdx.x == 0) {
    cycles[2 * blockIdx.x] = c1 - c0;
    cycles[2 * blockIdx.x + 1] = w1 - w0;
  }
}

}  // namespace

extern "C" {

int moe_calib_mfma(int blocks, int iters, uint32_t seed, int operands, int shape, float* sink,
                   unsigned long long* cycles, hipStream_t stream) {
  if (blocks <= 0 || iters <= 0 || (operands != 0 && operands != 1) ||
      (shape != 0 && shape != 1) || !sink || !cycles)
    return -1;
  if (shape == 0)
    hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(blocks), dim3(kWaves * 64), 0, stream, iters,
                       seed, operands, sink, cycles);
  else
    hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3(blocks), dim3(kWaves * 64), 0, stream, iters,
                       seed, operands, sink, cycles);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int moe_calib_wall_clock_khz(int* khz) {
  if (!khz) return -1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -5;
  return hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess ? 0 : -5;
}

}  // extern "C"
