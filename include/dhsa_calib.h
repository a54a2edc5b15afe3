/*
 * dhsa_calib.h - calibration kernels of libdhsa_calib.so (a separate library, not part of the DHSA
 * C ABI): they measure what one MI355X (gfx950) sustains for the two bounds the DHSA kernels are
 * reported against, so a roofline fraction can be read against a measured ceiling as well as the
 * published peak.  Every pointer is HIP device memory owned by the caller; calls are asynchronous
 * on `stream` (a hipStream_t, NULL = the default stream) and allocate nothing.  Return value: a
 * hipError_t code (0 = launched); arguments are checked before the launch.
 */
#ifndef DHSA_CALIB_H
#define DHSA_CALIB_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Dense bf16 matrix-core loop: `blocks` workgroups of 256 threads (4 waves; at most two workgroups
 * per CU are resident), each wave issuing 4 * iters independent v_mfma_f32_32x32x16_bf16
 * (32 * 32 * 16 * 2 FLOPs each) with no memory traffic in the loop.
 *   out  device float[blocks * 256]: one folded accumulator per thread (keeps the work live).
 * FLOPs per call: blocks * 4 * 4 * iters * 32768. */
int dhsa_calib_mfma_bf16(int blocks, int iters, float* out, void* stream);

/* Streaming read of `bytes` (a multiple of 16) from `src` by `blocks` workgroups of 256 threads,
 * each reading one contiguous range, 16 bytes per lane per load, eight loads in flight per lane.
 *   out  device float[blocks * 256]: one folded value per thread (keeps the loads live). */
int dhsa_calib_read(const void* src, size_t bytes, int blocks, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DHSA_CALIB_H */
