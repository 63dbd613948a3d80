// Internal interface between the C-ABI layer (api.cpp) and the HIP kernel files.
// Everything here has already been validated by api.cpp; launchers only compute grids and launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

constexpr int kHeadDim = 64;

// Packed varlen prefill. Strides in elements; the innermost (head_dim) stride is 1.
struct PrefillParams {
    const void* q;
    const void* k;
    const void* v;
    const float* sinks;
    const int32_t* cu_seqlens_q;
    const int32_t* cu_seqlens_k;
    void* out;
    int64_t q_stride_tok, q_stride_head;
    int64_t k_stride_tok, k_stride_head;
    int64_t v_stride_tok, v_stride_head;
    int64_t o_stride_tok, o_stride_head;
    int64_t total_q;     // Tq
    int64_t total_k;     // Tk
    int32_t num_seqs;    // B
    int32_t num_q_heads;
    int32_t num_kv_heads;
    float scale;
    int32_t causal;
    int32_t out_is_bf16;
    // Split-KV prefill (sinkattn_prefill_split) when partial_o is not null: split j of a sequence
    // covers keys [j * ks, min((j + 1) * ks, Lk)), ks = ceil(Lk / S) rounded up to 64; the state
    // of (token t, head h, split j) goes to row (t * Hq + h) * S + j of the contiguous partials.
    int32_t num_splits;
    float* partial_o;
    float* partial_m;
    float* partial_d;
};

// Split-KV decode of q_len tokens per sequence. q [B, T, Hq, D] (T = 1: [B, Hq, D]);
// k/v [B, Lcap, Hkv, D]; partials contiguous [B, T, Hq, C, D] / [B, T, Hq, C].
struct DecodeSplitParams {
    const void* q;
    const void* k;
    const void* v;
    const float* sinks;
    const int32_t* seqlens_k;
    float* partial_o;
    float* partial_m;
    float* partial_d;
    int64_t q_stride_b, q_stride_tok, q_stride_head;
    int64_t k_stride_b, k_stride_tok, k_stride_head;
    int64_t v_stride_b, v_stride_tok, v_stride_head;
    int64_t capacity;    // Lcap
    int64_t chunk_size;  // ceil(Lcap / C)
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t num_chunks;
    int32_t q_len;       // T >= 1 tokens per sequence, the last T of its seqlens_k keys
    float scale;
    // Fused split + merge only (sinkattn_decode): zero-initialised completion counters, one per
    // (sequence, KV head), and the merged outputs.
    uint32_t* counters;
    void* out;
    float* lse;          // may be null
    int64_t o_stride_b, o_stride_tok, o_stride_head;
    int64_t lse_stride_b, lse_stride_tok, lse_stride_head;
    int32_t out_is_bf16;
};

// Merge of rows (b, t, h): partials contiguous [batch, Hq, C, D] with batch = B x q_len; the
// output of row (b, t, h) sits at b * o_stride_b + t * o_stride_tok + h * o_stride_head.
struct DecodeMergeParams {
    const float* partial_o;
    const float* partial_m;
    const float* partial_d;
    void* out;
    float* lse;          // may be null
    int64_t o_stride_b, o_stride_tok, o_stride_head;
    int64_t lse_stride_b, lse_stride_tok, lse_stride_head;
    int32_t batch;
    int32_t q_len;
    int32_t num_q_heads;
    int32_t num_chunks;
    int32_t out_is_bf16;
};

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

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillParams& p, hipStream_t stream);
hipError_t launch_decode_split_bf16(const DecodeSplitParams& p, hipStream_t stream);
hipError_t launch_decode_split_f32(const DecodeSplitParams& p, hipStream_t stream);
// Split and merge in one launch (bf16); partials and counters as in DecodeSplitParams.
hipError_t launch_decode_fused_bf16(const DecodeSplitParams& p, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeMergeParams& p, hipStream_t stream);
hipError_t launch_moe_topk_softmax(const MoeTopkParams& p, hipStream_t stream);
hipError_t launch_gemm_bias(const GemmParams& p, bool fp8, hipStream_t stream);

}  // namespace sinkattn
