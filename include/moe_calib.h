/* Calibration of the bf16 MFMA roofline on the GPU in use (gfx950).
 *
 * For the measurement harness, not for the layer: the published dense bf16 peak assumes the
 * full shader clock, while under MFMA load the clock is set by the power limit and by the
 * data the multipliers see.  moe_calib_mfma runs every SIMD on nothing but independent
 * v_mfma_f32_32x32x16_bf16 instructions on register operands, so the rate it sustains (and
 * the clock it holds) is the ceiling an MFMA-bound kernel can approach on this GPU.  Built
 * into libmoe_calib.so, apart from the layer's library.
 */
#ifndef MOE_CALIB_H
#define MOE_CALIB_H

#include <stdint.h>

#include <hip/hip_runtime.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue one launch of `blocks` blocks (one per CU: pass the CU count to load the whole
 * chip) of 8 waves, each wave running `iters` iterations of 4 independent bf16 MFMAs:
 * shape 0 = v_mfma_f32_32x32x16_bf16 (blocks * 8 * iters * 4 * 32768 flops), shape 1 =
 * v_mfma_f32_16x16x32_bf16 (16384 flops each).  operands: 1 = random bf16 values (random
 * sign and mantissa, magnitudes in [0.25, 4), drawn from `seed`), 0 = all zeros.
 *   sink   device, float[blocks * 8]: each wave's sum of its accumulators (keeps the work).
 *   cycles device, uint64[2 * blocks]: per block, the shader-clock cycles and the
 *          constant-rate wall-clock ticks its first wave spent in the loop.
 * Returns 0, -1 on invalid arguments (nothing enqueued) or -5 if the launch failed. */
int moe_calib_mfma(int blocks, int iters, uint32_t seed, int operands, int shape, float* sink,
                   unsigned long long* cycles, hipStream_t stream);

/* Rate of the wall-clock counter of the current device, in kHz (0 on success). */
int moe_calib_wall_clock_khz(int* khz);

#ifdef __cplusplus
}
#endif

#endif /* MOE_CALIB_H */
