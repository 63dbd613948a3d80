// Internal interface between the C-ABI layer (api.cpp) and the MoE routing and linear-layer kernels.
// Everything here has already been validated by api.cpp; launchers only compute grids and launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

// MoE routing: logits [tokens, experts] (bf16 or f32, row stride in elements); per token the
// top_k expert ids (int32) and weights (bf16 or f32), rows of stride ids_stride / weights_stride.
struct MoeTopkParams {
    const void* logits;
    int32_t* ids;
    void* weights;
    int64_t logits_stride, ids_stride, weights_stride;
    int64_t tokens;
    int32_t experts;      // 1 .. 256
    int32_t top_k;        // 1 .. min(experts, 16)
    int32_t over_all;     // nonzero: normalise over all experts instead of the chosen K
    int32_t logits_is_bf16;
    int32_t weights_is_bf16;
    int32_t vector_rows;  // every logits row starts 16-byte aligned
};

// Linear layer with bias: y[m, n] = sum_k x[m, k] w[n, k] + bias[n]. bf16 x/w, or FP8 (E4M3)
// x/w with fp32 scales scale_x [M, K/128] and scale_w [ceil(N/128), K/128]. Row strides in
// elements; K a whole number of 64 (bf16) or 128 (FP8) steps.
struct GemmParams {
    const void* x;
    const void* w;
    const float* bias;     // may be null
    void* y;
    const float* scale_x;  // FP8 only
    const float* scale_w;  // FP8 only
    int64_t ldx, ldw, ldy;
    int64_t sx_stride_m, sx_stride_kb, sw_stride_nb, sw_stride_kb;
    int32_t m, n, k;
    int32_t y_is_bf16;
};

hipError_t launch_moe_topk_softmax(const MoeTopkParams& p, hipStream_t stream);
hipError_t launch_gemm_bias(const GemmParams& p, bool fp8, hipStream_t stream);

}  // namespace sinkattn
