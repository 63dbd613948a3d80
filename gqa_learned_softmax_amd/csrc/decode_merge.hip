// Log-sum-exp merge of split-KV chunk states (gfx950).
//
// Source: the split along the KV length in "GPT-OSS on Day 0" (Perplexity), section "Kernels for
// GPT-OSS", subsection "Sink attention", needs the per-chunk softmax states to be combined; the
// page names the split and the rule that only the first chunk carries the sink, and this is the
// standard combination of (max, scale, normalised output) states:
//   M = max_c m_c, w_c = d_c e^(m_c - M), out = sum_c w_c o_c / sum_c w_c, lse = M + ln sum_c w_c.
//
// One wave per (sequence, query head); lane = output channel d. Each chunk contributes one
// coalesced 256-byte row of partial_o.

#include "device_common.h"
#include "launch.h"

namespace sinkattn {
namespace {

constexpr int kMergeWaves = 4;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Chunks are taken 64 at a time: lane c loads (m_c, d_c) of its chunk, the wave agrees on the
// maximum, each lane forms its weight w_c, and lane d then accumulates w_c * o_c[d] with w_c
// broadcast from lane c (v_readlane). All loads of a 64-chunk block are independent, so they
// are in flight together.
__global__ __launch_bounds__(kMergeWaves * 64) void decode_merge_kernel(DecodeMergeParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t bh = static_cast<int64_t>(blockIdx.x) * kMergeWaves + (threadIdx.x >> 6);
    if (bh >= static_cast<int64_t>(p.batch) * p.num_q_heads) return;
    const int b = static_cast<int>(bh / p.num_q_heads);
    const int h = static_cast<int>(bh % p.num_q_heads);
    const int chunks = p.num_chunks;
    const float* pm = p.partial_m + bh * chunks;
    const float* pd = p.partial_d + bh * chunks;
    const float* po = p.partial_o + bh * chunks * kHeadDim;

    float big = kNegInf;
    for (int c0 = 0; c0 < chunks; c0 += 64) {
        const int c = c0 + lane;
        big = fmaxf(big, c < chunks ? pm[c] : kNegInf);
    }
    big = wave_max(big);
    float wsum = 0.0f, osum = 0.0f;
    if (big != kNegInf) {
        for (int c0 = 0; c0 < chunks; c0 += 64) {
            const int c = c0 + lane;
            float w = 0.0f;
            if (c < chunks) {
                const float mc = pm[c];
                w = mc == kNegInf ? 0.0f : pd[c] * expf(mc - big);
            }
            wsum += w;
            const int n = chunks - c0 < 64 ? chunks - c0 : 64;
            const float* rows = po + static_cast<int64_t>(c0) * kHeadDim + lane;
            int j = 0;
            for (; j + 8 <= n; j += 8) {
                float o[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) o[u] = rows[static_cast<int64_t>(j + u) * kHeadDim];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    osum = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j + u)), o[u], osum);
            }
            for (; j < n; ++j)
                osum = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j)),
                            rows[static_cast<int64_t>(j) * kHeadDim], osum);
        }
        wsum = wave_sum(wsum);
    }
    const float o = wsum > 0.0f ? osum / wsum : 0.0f;
    const int64_t off = b * p.o_stride_b + h * p.o_stride_head + lane;
    if (p.out_is_bf16)
        static_cast<__bf16*>(p.out)[off] = (__bf16)o;
    else
        static_cast<float*>(p.out)[off] = o;
    if (p.lse != nullptr && lane == 0)
        p.lse[b * p.lse_stride_b + h * p.lse_stride_head] = wsum > 0.0f ? big + logf(wsum) : kNegInf;
}

}  // namespace

hipError_t launch_decode_merge(const DecodeMergeParams& p, hipStream_t stream) {
    const int64_t rows = static_cast<int64_t>(p.batch) * p.num_q_heads;
    const int64_t blocks = (rows + kMergeWaves - 1) / kMergeWaves;
    decode_merge_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(kMergeWaves * 64), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace sinkattn
