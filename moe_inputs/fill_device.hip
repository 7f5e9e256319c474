// Device fill of seeded synthetic inputs (test and benchmark infrastructure).
// Values are defined in philox_normal.h; a host build of the same header gives the
// same bits, so inputs made here can be regenerated slice by slice on the host.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "philox_normal.h"

__global__ void __launch_bounds__(256) fill_f32(float* out, uint64_t start, uint64_t count,
                                                uint32_t seed, uint32_t tid, float scale) {
  uint64_t n = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (; n < count; n += stride) out[n] = moe_inputs_value_f32(start + n, seed, tid, scale);
}

__global__ void __launch_bounds__(256) fill_bf16(uint16_t* out, uint64_t start, uint64_t count,
                                                 uint32_t seed, uint32_t tid, float scale) {
  uint64_t n = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (; n < count; n += stride)
    out[n] = moe_inputs_bf16_rne(moe_inputs_value_f32(start + n, seed, tid, scale));
}

// Returns 0 on success, the hipError_t value otherwise.
extern "C" int moe_inputs_fill_device(void* out, int is_bf16, uint64_t start, uint64_t count,
                                      uint32_t seed, uint32_t tensor_id, float scale,
                                      hipStream_t stream) {
  if (count == 0) return 0;
  uint64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (is_bf16)
    fill_bf16<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>((uint16_t*)out, start, count,
                                                                seed, tensor_id, scale);
  else
    fill_f32<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>((float*)out, start, count, seed,
                                                               tensor_id, scale);
  return (int)hipGetLastError();
}
