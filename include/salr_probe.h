/*
 * salr_probe.h - measurement probes of libsalr.so: the achievable HBM read
 * rate and bf16 matrix-core rate of the GPU the library runs on, measured
 * with kernels of the same shape as the SALR forward's (wave64, 16-byte
 * lane loads, v_mfma bf16 instructions).  The forward's roofline fractions
 * are reported against these measured peaks beside the vendor peaks
 * (8 TB/s HBM, 2.5 PFLOP/s dense bf16).
 *
 * Both calls are asynchronous on `stream` (a hipStream_t passed as void*,
 * NULL = null stream); the caller times them with events on that stream.
 * The library allocates nothing.  Return value: 0 (SALR_OK), or
 * SALR_ERR_INVALID_ARG / SALR_ERR_HIP as in salr.h.
 */
#ifndef SALR_PROBE_H_
#define SALR_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * salr_probe_stream_read - read `bytes` of device memory at `src` once, with
 * 16-byte lane loads spread over `workgroups` workgroups of 512 threads
 * (contiguous 8 KB blocks per workgroup step).  Each workgroup folds what it
 * read into one word of `sink` (device, at least `workgroups` uint32), so
 * the loads cannot be dropped.  src must be 16-byte aligned and bytes a
 * multiple of 16; workgroups in [1, 65536].
 */
int salr_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream);

/*
 * salr_probe_mfma - run `iters` rounds of independent bf16 matrix-core
 * instructions in every wave of `workgroups` workgroups of 256 threads
 * (4 waves, one per SIMD of a CU).  shape 0: v_mfma_f32_16x16x32_bf16,
 * 8 accumulator chains per wave (8 x 16384 flop per round);
 * shape 1: v_mfma_f32_32x32x16_bf16, 4 chains (4 x 32768 flop per round).
 * Flop per call = workgroups * 4 * iters * 131072.  The accumulators are
 * folded into out[workgroup] (device, at least `workgroups` floats).
 * iters in [1, 2^24], workgroups in [1, 65536].
 */
int salr_probe_mfma(float* out, int32_t workgroups, int32_t iters, int32_t shape, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SALR_PROBE_H_ */
