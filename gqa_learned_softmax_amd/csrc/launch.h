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

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillParams& p, hipStream_t stream);
hipError_t launch_decode_split_bf16(const DecodeSplitParams& p, hipStream_t stream);
hipError_t launch_decode_split_f32(const DecodeSplitParams& p, hipStream_t stream);
// Split and merge in one launch (bf16); partials and counters as in DecodeSplitParams.
hipError_t launch_decode_fused_bf16(const DecodeSplitParams& p, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeMergeParams& p, hipStream_t stream);

// sinkattn_decode_static: the library-owned workspace, one per GPU (static_workspace.hip).
constexpr size_t kStaticWorkspaceBytes = size_t(32) << 20;
// Device address of the current device's copy; the first call on a device looks it up and clears
// it with a kernel on `stream`.
hipError_t static_decode_workspace(hipStream_t stream, void** out);

}  // namespace sinkattn
