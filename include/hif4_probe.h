/*
 * hif4_probe.h -- C ABI of libhif4_probe.so: measurement probes for the
 * rooflines the benchmark reports against. Not part of the HiF4 method and
 * not linked into libhif4.so.
 */
#ifndef HIF4_PROBE_H
#define HIF4_PROBE_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * hif4_probe_mfma_bf16 -- the achievable dense bf16 matrix-core rate under a
 * full-chip load: `blocks` workgroups of 4 waves, each wave issuing `iters` x
 * 16 v_mfma_f32_32x32x16_bf16 (32,768 flops each) back to back from
 * registers. out: fp32 [blocks * 256] device buffer (one sum per thread, so
 * that nothing is optimized away). Asynchronous on `stream`.
 * Returns 0, 1 for a bad argument, 7 if the launch failed.
 */
__attribute__((visibility("default"))) int hif4_probe_mfma_bf16(int blocks, int iters, float *out,
                                                                 hipStream_t stream);

/*
 * hif4_probe_copy -- the achievable HBM streaming rate: copies `bytes`
 * (a multiple of 16) from src to dst (device buffers, not overlapping) with a
 * grid-stride kernel of `blocks` workgroups of 256 threads, 16-byte
 * non-temporal loads and stores, four loads in flight per lane.
 * Returns 0, 1 for a bad argument, 7 if the launch failed.
 */
__attribute__((visibility("default"))) int hif4_probe_copy(const void *src, void *dst, size_t bytes,
                                                            int blocks, hipStream_t stream);

/*
 * hif4_probe_read -- the achievable HBM read rate: reads `bytes` (a multiple
 * of 16) of src with the same grid-stride pattern as hif4_probe_copy and
 * writes one u32 per thread to out (u32 [blocks * 256]).
 * Returns 0, 1 for a bad argument, 7 if the launch failed.
 */
__attribute__((visibility("default"))) int hif4_probe_read(const void *src, size_t bytes, void *out,
                                                            int blocks, hipStream_t stream);

/*
 * hif4_probe_read4_write1 -- the achievable HBM rate for the quantizer's
 * traffic mix: reads `src_bytes` (a multiple of 64) of src and writes
 * src_bytes / 4 to dst (device buffers, not overlapping): lane i loads word
 * i of each quarter of src (16-byte non-temporal loads) and stores their XOR
 * to word i of dst, with a grid-stride kernel of `blocks` workgroups of 256
 * threads.
 * Returns 0, 1 for a bad argument, 7 if the launch failed.
 */
__attribute__((visibility("default"))) int hif4_probe_read4_write1(const void *src,
                                                                    size_t src_bytes, void *dst,
                                                                    int blocks,
                                                                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HIF4_PROBE_H */
