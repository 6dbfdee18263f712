/*
 * dsa_probe.h - achievable-peak probes for MI355X (gfx950), used to state
 * roofline fractions against measured as well as published peaks.  Not part
 * of the DSA path (libdsa.so); built as libdsa_probe.so.
 *
 * Every call launches one kernel, asynchronously, on `stream` (a hipStream_t;
 * NULL = the default stream) and returns 0, or -1 for invalid arguments
 * (nothing launched).  Time the launches with events on the same stream.
 * Pointers are device memory owned by the caller.
 *
 * dsa_probe_mfma: `blocks` workgroups of 256 threads; every wave issues
 *   `iters` (even) rounds of 8 independent matrix instructions of `kind`:
 *     0  v_mfma_scale_f32_16x16x128_f8f6f4 (e4m3 x e4m3, 65536 FLOP each)
 *     1  v_mfma_f32_16x16x32_bf16  (16384 FLOP each)
 *     2  v_mfma_f32_32x32x16_bf16  (32768 FLOP each)
 *   and writes one float per thread to sink[blocks * 256] (so the work is
 *   kept).  dsa_probe_mfma_flops() returns the FLOPs one such launch does.
 * dsa_probe_read: streams `bytes` (a multiple of 16 * 256 * 8 * blocks)
 *   from `buf` (16-byte aligned): workgroup b of `blocks` reads the b-th
 *   contiguous 1/blocks of the buffer with 16-byte non-temporal loads, eight
 *   in flight per thread, and writes one float per thread to
 *   sink[blocks * 256].  Returns -1 for sizes that do not divide.
 */
#ifndef DSA_PROBE_H_
#define DSA_PROBE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int dsa_probe_mfma(int kind, int64_t iters, int64_t blocks, float* sink, void* stream);
double dsa_probe_mfma_flops(int kind, int64_t iters, int64_t blocks);
int dsa_probe_read(const void* buf, int64_t bytes, int64_t blocks, float* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_PROBE_H_ */
