// Log-sum-exp merge of split-KV chunk states (gfx950): the combination rule of chunk_merge.h
// (section "Kernels for GPT-OSS", subsection "Sink attention", of "GPT-OSS on Day 0") as a kernel
// of its own. One wave per (sequence, token, query head); lane = output channel d. Each chunk
// contributes one coalesced 256-byte row of partial_o.

#include "chunk_merge.h"
#include "device_common.h"
#include "launch.h"

namespace sinkattn {
namespace {

constexpr int kMergeWaves = 4;

__global__ __launch_bounds__(kMergeWaves * 64) void decode_merge_kernel(DecodeMergeParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t bh = static_cast<int64_t>(blockIdx.x) * kMergeWaves + (threadIdx.x >> 6);
    if (bh >= static_cast<int64_t>(p.batch) * p.num_q_heads) return;
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
    const int64_t rows = static_cast<int64_t>(p.batch) * p.num_q_heads;
    const int64_t blocks = (rows + kMergeWaves - 1) / kMergeWaves;
    decode_merge_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(kMergeWaves * 64), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace sinkattn
