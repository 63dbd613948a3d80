// Log-sum-exp combination of split-KV chunk states, one wave per (sequence, query head).
//
// Source: the split along the KV length in "GPT-OSS on Day 0" (Perplexity), section "Kernels for
// GPT-OSS", subsection "Sink attention", needs the per-chunk softmax states to be combined; the
// page names the split and the rule that only the first chunk carries the sink, and this is the
// standard combination of (max, scale, normalised output) states:
//   M = max_c m_c, w_c = d_c e^(m_c - M), out = sum_c w_c o_c / sum_c w_c, lse = M + ln sum_c w_c.
// Used by the stand-alone merge kernel and by the last work-group of the fused decode kernel.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace sinkattn {

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

// Combines `chunks` states of one row: pm/pd hold (m_c, d_c) (natural-log m), po holds the
// normalised chunk outputs o_c as `chunks` rows of kHeadDim floats. Lane d of the calling wave
// receives out[d]; `lse` is the same in every lane. The calling wave must have all 64 lanes
// active. With more than 16 chunks they are taken 64 at a time: lane c loads
// (m_c, d_c), the wave agrees on the maximum, each lane forms its weight w_c, and lane d then
// accumulates w_c * o_c[d] with w_c broadcast from lane c (v_readlane). The loads of a block are
// independent of each other, so they are in flight together; with at most 64 chunks the states
// are loaded once.
__device__ __forceinline__ void merge_chunk_states(const float* pm, const float* pd, const float* po,
                                                   int chunks, int lane, float& out, float& lse) {
    if (chunks <= 16) {
        // Few chunks: every load of the row (m_c, d_c on lanes c, and o_c[lane] for all c) is
        // issued before any of them is used, so the row costs one memory round trip, not two.
        float o[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) o[c] = c < chunks ? po[static_cast<int64_t>(c) * kHeadDim + lane] : 0.0f;
        const float mc = lane < chunks ? pm[lane] : kNegInf;
        const float dc = lane < chunks ? pd[lane] : 0.0f;
        float big = mc;
#pragma unroll
        for (int x = 8; x > 0; x >>= 1) big = fmaxf(big, __shfl_xor(big, x));
        big = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(big), 0));
        const float w = mc == kNegInf ? 0.0f : dc * expf(mc - big);
        float wsum = w;
#pragma unroll
        for (int x = 8; x > 0; x >>= 1) wsum += __shfl_xor(wsum, x);
        wsum = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsum), 0));
        float osum = 0.0f;
#pragma unroll
        for (int c = 0; c < 16; ++c)
            if (c < chunks) osum = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), c)), o[c], osum);
        out = wsum > 0.0f ? osum / wsum : 0.0f;
        lse = wsum > 0.0f ? big + logf(wsum) : kNegInf;
        return;
    }
    const float m_first = lane < chunks ? pm[lane] : kNegInf;
    const float d_first = lane < chunks ? pd[lane] : 0.0f;
    float big = m_first;
    for (int c = 64 + lane; c - lane < chunks; c += 64) big = fmaxf(big, c < chunks ? pm[c] : kNegInf);
    big = wave_max(big);
    float wsum = 0.0f, osum = 0.0f;
    if (big != kNegInf) {
        for (int c0 = 0; c0 < chunks; c0 += 64) {
            const int c = c0 + lane;
            const float mc = c0 == 0 ? m_first : (c < chunks ? pm[c] : kNegInf);
            const float dc = c0 == 0 ? d_first : (c < chunks ? pd[c] : 0.0f);
            const float w = mc == kNegInf ? 0.0f : dc * expf(mc - big);
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
    out = wsum > 0.0f ? osum / wsum : 0.0f;
    lse = wsum > 0.0f ? big + logf(wsum) : kNegInf;
}

// Four rows per wave: the same combination with each 16-lane quarter of the wave on its own row
// (pm/pd/po of the calling lane's row). Lane j of a quarter loads (m_c, d_c) of chunks c = j,
// j + 16, ..., and channels 4j .. 4j + 3 of every chunk's o (16-byte loads), so a wave has the
// loads of four rows in flight at once; weights are broadcast inside the quarter. Rows with many
// more chunks than 16 are better served by merge_chunk_states.
__device__ __forceinline__ void merge_chunk_states_x4(const float* pm, const float* pd, const float* po,
                                                      int chunks, int lane, f32x4& out, float& lse) {
    const int j = lane & 15;
    const int quarter = lane & 48;
    float big = kNegInf;
    for (int c = j; c - j < chunks; c += 16) big = fmaxf(big, c < chunks ? pm[c] : kNegInf);
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) big = fmaxf(big, __shfl_xor(big, o));
    float wsum = 0.0f;
    f32x4 osum = zero_f32x4();
    if (big != kNegInf) {
        for (int c0 = 0; c0 < chunks; c0 += 16) {
            const int c = c0 + j;
            const float mc = c < chunks ? pm[c] : kNegInf;
            const float w = mc == kNegInf ? 0.0f : pd[c] * expf(mc - big);
            wsum += w;
            const int n = chunks - c0 < 16 ? chunks - c0 : 16;
            const float* rows = po + static_cast<int64_t>(c0) * kHeadDim + 4 * j;
            int u = 0;
            for (; u + 4 <= n; u += 4) {
                f32x4 o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = *reinterpret_cast<const f32x4*>(rows + (u + e) * kHeadDim);
#pragma unroll
                for (int e = 0; e < 4; ++e) osum += __shfl(w, quarter + u + e) * o[e];
            }
            for (; u < n; ++u)
                osum += __shfl(w, quarter + u) * *reinterpret_cast<const f32x4*>(rows + u * kHeadDim);
        }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) wsum += __shfl_xor(wsum, o);
    }
    out = wsum > 0.0f ? osum / wsum : zero_f32x4();
    lse = wsum > 0.0f ? big + logf(wsum) : kNegInf;
}

// Four rows per wave with at most 16 chunks: as merge_chunk_states_x4, but every load of a row
// (m_c, d_c on lanes c of the quarter, and channels 4j .. 4j + 3 of every o_c) is issued before any
// is used, so a row costs one memory round trip. The 16 lanes of a calling quarter must be active
// together.
__device__ __forceinline__ void merge_few_chunk_states_x4(const float* pm, const float* pd, const float* po,
                                                          int chunks, int lane, f32x4& out, float& lse) {
    const int j = lane & 15;
    const int quarter = lane & 48;
    f32x4 o[16];
#pragma unroll
    for (int c = 0; c < 16; ++c)
        o[c] = c < chunks ? *reinterpret_cast<const f32x4*>(po + c * kHeadDim + 4 * j) : zero_f32x4();
    const float mc = j < chunks ? pm[j] : kNegInf;
    const float dc = j < chunks ? pd[j] : 0.0f;
    float big = mc;
#pragma unroll
    for (int x = 8; x > 0; x >>= 1) big = fmaxf(big, __shfl_xor(big, x));
    const float w = mc == kNegInf ? 0.0f : dc * expf(mc - big);
    float wsum = w;
#pragma unroll
    for (int x = 8; x > 0; x >>= 1) wsum += __shfl_xor(wsum, x);
    f32x4 osum = zero_f32x4();
#pragma unroll
    for (int c = 0; c < 16; ++c)
        if (c < chunks) osum += __shfl(w, quarter + c) * o[c];
    out = wsum > 0.0f ? osum / wsum : zero_f32x4();
    lse = wsum > 0.0f ? big + logf(wsum) : kNegInf;
}

}  // namespace sinkattn
