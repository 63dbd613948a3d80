// Log-sum-exp merge of split-KV chunk states (gfx950): the combination rule of chunk_merge.h
// (section "Kernels for GPT-OSS", subsection "Sink attention", of "GPT-OSS on Day 0") as a kernel
// of its own. One wave per (sequence, token, query head), lane = output channel d; each chunk
// contributes one coalesced 256-byte row of partial_o. With many rows (>= 8192) and at most 16
// chunks, four rows per wave instead (16 lanes and 4 channels per lane, all loads of a row issued at
// once): fewer, fuller waves, measured faster there and slower on a few hundred rows.

#include "chunk_merge.h"
#include "device_common.h"
#include "launch.h"
#include "plan.h"

namespace sinkattn {
namespace {

// Four rows per wave (chunks <= 16). Rows past the end are clamped to the last row and not
// written, so every lane stays active for the quarter reductions.
__global__ __launch_bounds__(kMergeWaves * 64) void decode_merge_x4_kernel(DecodeMergeParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t rows = static_cast<int64_t>(p.batch) * p.num_q_heads;
    const int64_t bh_raw = (static_cast<int64_t>(blockIdx.x) * kMergeWaves + (threadIdx.x >> 6)) * 4 + (lane >> 4);
    const bool valid = bh_raw < rows;
    const int64_t bh = valid ? bh_raw : rows - 1;
    const int64_t bt = bh / p.num_q_heads;
    const int b = static_cast<int>(bt / p.q_len);
    const int tok = static_cast<int>(bt % p.q_len);
    const int h = static_cast<int>(bh % p.num_q_heads);
    const int chunks = p.num_chunks;
    f32x4 o;
    float lse;
    merge_few_chunk_states_x4(p.partial_m + bh * chunks, p.partial_d + bh * chunks,
                              p.partial_o + bh * chunks * kHeadDim, chunks, lane, o, lse);
    if (!valid) return;
    const int64_t off = b * p.o_stride_b + tok * p.o_stride_tok + h * p.o_stride_head + 4 * (lane & 15);
    if (p.out_is_bf16) {
        bf16x4 ob;
#pragma unroll
        for (int e = 0; e < 4; ++e) ob[e] = (__bf16)o[e];
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.out) + off) = ob;
    } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + off) = o;
    }
    if (p.lse != nullptr && (lane & 15) == 0)
        p.lse[b * p.lse_stride_b + tok * p.lse_stride_tok + h * p.lse_stride_head] = lse;
}

// One row per wave. Work-group order: work-groups go to the eight XCDs round-robin by index, and
// when the rows come in whole groups of 8 blocks of 16, work-group w merges quarter (w / 8) % 4 of
// 16-row block 8 (w / 32) + w % 8, so block j is merged on XCD j mod 8. A split launch of a single
// round whose work-groups each cover 16 consecutive rows (two KV heads of a group of 8, one token)
// writes block j's chunk states from XCD j mod 8 too, so each block is merged on the XCD that wrote
// it: 8 x 8192 keys, 64/8 heads, split + merge 26.5 instead of 27.2 us (same machine). The merge's
// L2 misses (FETCH_SIZE) are the same in either order, so the states do not come from that L2; why
// the aligned order is faster is not established. For other split layouts this order is as good as
// the plain one.
__global__ __launch_bounds__(kMergeWaves * 64) void decode_merge_kernel(DecodeMergeParams p) {
    static_assert(kMergeWaves == 4, "four work-groups per 16-row block");
    const int lane = threadIdx.x & 63;
    const int64_t rows = static_cast<int64_t>(p.batch) * p.num_q_heads;
    const int64_t w = blockIdx.x;
    const int64_t bh = (rows % 128 == 0 ? 16 * (8 * (w / 32) + w % 8) + 4 * ((w / 8) % 4) : 4 * w) + (threadIdx.x >> 6);
    if (bh >= rows) return;
    const int64_t bt = bh / p.num_q_heads;
    const int b = static_cast<int>(bt / p.q_len);
    const int tok = static_cast<int>(bt % p.q_len);
    const int h = static_cast<int>(bh % p.num_q_heads);
    const int chunks = p.num_chunks;
    float o, lse;
    merge_chunk_states(p.partial_m + bh * chunks, p.partial_d + bh * chunks,
                       p.partial_o + bh * chunks * kHeadDim, chunks, lane, o, lse);
    const int64_t off = b * p.o_stride_b + tok * p.o_stride_tok + h * p.o_stride_head + lane;
    if (p.out_is_bf16)
        static_cast<__bf16*>(p.out)[off] = (__bf16)o;
    else
        static_cast<float*>(p.out)[off] = o;
    if (p.lse != nullptr && lane == 0)
        p.lse[b * p.lse_stride_b + tok * p.lse_stride_tok + h * p.lse_stride_head] = lse;
}

}  // namespace

hipError_t launch_decode_merge(const DecodeMergeParams& p, hipStream_t stream) {
    const Launch l = plan_decode_merge(p);
    if (merge_four_rows_per_wave(p))
        decode_merge_x4_kernel<<<dim3(static_cast<unsigned>(l.grid)), dim3(l.block), 0, stream>>>(p);
    else
        decode_merge_kernel<<<dim3(static_cast<unsigned>(l.grid)), dim3(l.block), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace sinkattn
