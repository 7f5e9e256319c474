/*
 * Host fill of seeded synthetic inputs (test and benchmark infrastructure).
 * Values are defined in philox_normal.h; this file only loops over indices.
 */
#include <stddef.h>
#include <stdint.h>
#include "philox_normal.h"

/* out: float[count] (is_bf16 == 0) or uint16 bf16 bits[count] (is_bf16 != 0); element n
 * gets the value of tensor index start + n. */
void moe_inputs_fill_host(void* out, int is_bf16, uint64_t start, uint64_t count,
                          uint32_t seed, uint32_t tensor_id, float scale) {
  if (is_bf16) {
    uint16_t* o = (uint16_t*)out;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < (int64_t)count; ++n)
      o[n] = moe_inputs_bf16_rne(moe_inputs_value_f32(start + (uint64_t)n, seed, tensor_id, scale));
  } else {
    float* o = (float*)out;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < (int64_t)count; ++n)
      o[n] = moe_inputs_value_f32(start + (uint64_t)n, seed, tensor_id, scale);
  }
}

/* Widen bf16 bits to fp32 (exact). */
void moe_inputs_bf16_to_f32(const uint16_t* in, float* out, uint64_t count) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < (int64_t)count; ++n) {
    union { uint32_t u; float f; } b;
    b.u = (uint32_t)in[n] << 16;
    out[n] = b.f;
  }
}
