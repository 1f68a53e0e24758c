/*
 * Peak calibration (measurement only, built as libpdllm_calib.so): the dense
 * bf16 MFMA rate and the HBM read and copy rates this GPU reaches in
 * practice.  The benchmark reports every roofline fraction against both the
 * published MI355X peaks and these measured ceilings.  Nothing on the
 * attention path calls these functions.  All pointers are device pointers
 * owned by the caller; every call is asynchronous on `stream` (time it with
 * events on that stream) and returns a hipError_t value (0 on success).
 */
#ifndef PDLLM_CALIB_H_
#define PDLLM_CALIB_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* n_wg workgroups of 4 wavefronts, each running `iters` rounds of four
 * independent v_mfma_f32_32x32x16_bf16 chains on full-entropy bf16 operands
 * (the MFMA rate depends on the data).  sink: device float[n_wg * 256]. */
int pdllm_calib_mfma_bf16(int64_t iters, int32_t n_wg, float* sink, void* stream);
/* FLOPs of one pdllm_calib_mfma_bf16 call (host function). */
int64_t pdllm_calib_mfma_bf16_flops(int64_t iters, int32_t n_wg);

/* Read `bytes` (a multiple of 16, buf 16-byte aligned) once: workgroup w of
 * n_wg (256 threads each) streams the w-th contiguous block in 16-byte loads,
 * four in flight per thread; an XOR of the data goes to sink (device
 * uint32_t[n_wg * 256]) so no load is dropped. */
int pdllm_calib_hbm_read(const void* buf, int64_t bytes, int32_t n_wg, uint32_t* sink, void* stream);

/* Copy `bytes` from src to dst (both 16-byte aligned, not overlapping), in
 * the same blocks as pdllm_calib_hbm_read. */
int pdllm_calib_hbm_copy(const void* src, void* dst, int64_t bytes, int32_t n_wg, void* stream);

#ifdef __cplusplus
}
#endif

#endif  /* PDLLM_CALIB_H_ */
