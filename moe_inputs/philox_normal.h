/*
 * Seeded synthetic input values for the MoE layer workloads (test and benchmark
 * infrastructure; none of the layer's arithmetic lives here).
 *
 * One value per element index i of a tensor:
 *   1. Philox4x32-10 (Salmon, Moraes, Dror, Shaw: "Parallel random numbers: as easy as
 *      1, 2, 3", SC'11) with key (seed, tensor_id) and counter (lo32(i), hi32(i), 0, 0)
 *      gives four 32-bit words.
 *   2. The words are split into eight 16-bit uniforms u_0..u_7 on {0..65535}; their sum
 *      minus 8*32767.5 = 262140 is an exact integer S (Irwin-Hall approximation of a
 *      normal, n = 8; |S| <= 262140).
 *   3. value = (float)S * scale, one correctly rounded fp32 multiply.  The caller picks
 *      scale = std / sqrt(8 * (2^32 - 1) / 12), rounded once to fp32.
 *   4. For bf16 tensors the fp32 value is rounded to nearest-even bf16 with integer ops.
 * Every step is integer or a single IEEE multiply, so a host build and a device build
 * of this header give bit-identical values.
 */
#ifndef MOE_INPUTS_PHILOX_NORMAL_H
#define MOE_INPUTS_PHILOX_NORMAL_H

#include <stdint.h>

#if defined(__HIPCC__)
#define MOE_INPUTS_HD __host__ __device__ static inline
#else
#define MOE_INPUTS_HD static inline
#endif

MOE_INPUTS_HD void moe_inputs_philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)M0 * (uint64_t)c[0];
    uint64_t p1 = (uint64_t)M1 * (uint64_t)c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k0;
    uint32_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += W0;
    k1 += W1;
  }
}

/* Exact integer S for element index i (see step 2 above). */
MOE_INPUTS_HD int32_t moe_inputs_irwin_hall8(uint64_t i, uint32_t seed, uint32_t tensor_id) {
  uint32_t c[4] = {(uint32_t)i, (uint32_t)(i >> 32), 0u, 0u};
  moe_inputs_philox4x32_10(c, seed, tensor_id);
  int32_t s = 0;
  for (int w = 0; w < 4; ++w) s += (int32_t)(c[w] & 0xFFFFu) + (int32_t)(c[w] >> 16);
  return s - 262140;
}

MOE_INPUTS_HD float moe_inputs_value_f32(uint64_t i, uint32_t seed, uint32_t tensor_id,
                                         float scale) {
  float s = (float)moe_inputs_irwin_hall8(i, seed, tensor_id);
  return s * scale;
}

/* Round-to-nearest-even fp32 -> bf16 bit pattern (finite inputs only). */
MOE_INPUTS_HD uint16_t moe_inputs_bf16_rne(float v) {
  union { float f; uint32_t u; } b;
  b.f = v;
  uint32_t u = b.u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

#endif
