/* libsinkattn_ceilings: measured hardware ceilings, for reporting only.
 *
 * Kernels that bound what the attention kernels of libsinkattn can reach on the GPU that runs
 * them: a streaming read of HBM (the bound of the split-KV decode, which reads every K/V byte once),
 * a loop of bf16 matrix-core instructions (the bound of the prefill's two products), and loops of
 * the prefill's inner-loop instructions that give what each costs a SIMD. The benchmark divides the
 * attention kernels' rates by these measured rates, beside the published peaks. Nothing in
 * libsinkattn depends on this library.
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

/* The split-KV decode's read pattern alone: `k` and `v` (device, 16-byte aligned) each hold
 * seqs x chunks x rows_per_chunk rows of `row_bytes` bytes (a multiple of 256), row-major; every
 * 256-byte slice of every row of both is read once with non-temporal 16-byte loads, by
 * seqs x chunks x (row_bytes / 256) work-groups of 512 threads, one per (slice, sequence, chunk)
 * numbered slice fastest, then sequence, then chunk (the decode kernel's order for pairs of KV heads
 * of 128 bytes each). `out4` as above. */
int sinkattn_ceiling_stream_read_slices(const void* k, const void* v, int seqs, int chunks, int rows_per_chunk,
                                        int row_bytes, void* out4, void* stream);

/* `blocks` work-groups of four waves, each wave issuing `iters` x 4 independent
 * v_mfma_f32_32x32x16_bf16; `out4` as above. */
int sinkattn_ceiling_mfma_bf16(int blocks, int iters, void* out4, void* stream);

/* Floating-point operations of one sinkattn_ceiling_mfma_bf16(blocks, iters) launch. */
double sinkattn_ceiling_mfma_bf16_flop(int blocks, int iters);

/* As sinkattn_ceiling_mfma_bf16, on random bf16 operands (four A and four B per lane, uniform in
 * [-2, 2), cycled so consecutive MFMAs share none), 8 MFMAs per wave and iteration: the MFMA rate at
 * the clock the chip holds when the operand bits switch as real data's do. */
int sinkattn_ceiling_mfma_bf16_random(int blocks, int iters, void* out4, void* stream);

/* Floating-point operations of one sinkattn_ceiling_mfma_bf16_random(blocks, iters) launch. */
double sinkattn_ceiling_mfma_bf16_random_flop(int blocks, int iters);

/* `blocks` work-groups of four waves, each wave repeating `iters` times one group of instructions
 * (independent of recent results except in kind 7), by `kind`: 0: 16 v_exp_f32; 1: 16 v_mul_f32;
 * 2: 16 v_cvt_pk_bf16_f32; 3: 16 v_fma_f32; 4: 4 v_mfma_f32_32x32x16_bf16; 5: 4
 * v_mfma_f32_16x16x32_bf16; 6: 4 of kind 4 with 4 v_exp_f32 after each; 7: 8
 * v_mfma_f32_32x32x16_bf16, 2 v_mfma_f32_16x16x32_bf16, 16 v_exp_f32, 16 v_mul_f32 and 8
 * v_cvt_pk_bf16_f32 interleaved, each exponential taking a product and each pack two exponentials
 * (a quarter of a prefill tile's instructions per wave). `clk` is a device buffer of 2 x `blocks`
 * uint64 that receives, per work-group, the shader-clock cycles (s_memtime) and 100 MHz ticks
 * (s_memrealtime) of wave 0's loop. `out4` as above. */
int sinkattn_ceiling_issue(int kind, int blocks, int iters, void* clk, void* out4, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SINKATTN_CEILINGS_H */
