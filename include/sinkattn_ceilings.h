/* libsinkattn_ceilings: measured hardware ceilings, for reporting only.
 *
 * Two kernels that bound what the attention kernels of libsinkattn can reach on the GPU that runs
 * them: a streaming read of HBM (the bound of the split-KV decode, which reads every K/V byte once)
 * and a loop of bf16 matrix-core instructions (the bound of the prefill's two products). The
 * benchmark divides the attention kernels' rates by these measured rates, beside the published
 * peaks. Nothing in libsinkattn depends on this library.
 *
 * Ownership and errors: the caller owns every buffer (device memory); the calls launch one kernel
 * on `stream` (a hipStream_t, NULL for the default stream), never synchronise, allocate nothing, and
 * return 0 on success, 1 for an invalid argument (nothing launched) and 2 if the launch failed.
 */
#ifndef SINKATTN_CEILINGS_H
#define SINKATTN_CEILINGS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads all `bytes` bytes of device buffer `buf` (16-byte aligned, `bytes` a multiple of 16) once,
 * with `blocks` work-groups of 256 threads and non-temporal 16-byte loads. `out4` is a device
 * pointer to 4 writable bytes that the kernel writes only for a fill pattern no caller uses. */
int sinkattn_ceiling_stream_read(const void* buf, uint64_t bytes, int blocks, void* out4, void* stream);

/* `blocks` work-groups of four waves, each wave issuing `iters` x 4 independent
 * v_mfma_f32_32x32x16_bf16; `out4` as above. */
int sinkattn_ceiling_mfma_bf16(int blocks, int iters, void* out4, void* stream);

/* Floating-point operations of one sinkattn_ceiling_mfma_bf16(blocks, iters) launch. */
double sinkattn_ceiling_mfma_bf16_flop(int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif /* SINKATTN_CEILINGS_H */
