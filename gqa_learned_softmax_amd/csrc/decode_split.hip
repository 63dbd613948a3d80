// Split-KV decode with a learned per-head softmax sink (gfx950).
//
// Source: "GPT-OSS on Day 0" (Perplexity), section "Kernels for GPT-OSS", subsection "Sink
// attention": attention is parallelised over heads and over the KV length; the online softmax
// keeps a running max m and running scale d per query row, m starts at the head's sink value and
// d at 1, and when the KV length is split into chunks the sink is counted in the first chunk only.
//
// Work decomposition: one work-group per (sequence b, KV head g, chunk c). The G = Hq/Hkv query
// heads that share KV head g are the 16 columns of the matrix-core tiles (columns >= G are
// padding), so every K/V byte is read from HBM once and used by all G heads. Inside the
// work-group, four waves take interleaved 32-key blocks of the chunk and keep their own softmax
// state; the states are merged through LDS at the end and written as the chunk's (m, d, o).
//
// Per 64-key block, per wave (the next block's loads are in flight meanwhile):
//   S^T (64 keys x 16 heads) = K (64 x 64) . Q^T (64 x 16): 8 MFMA 16x16x32, K straight from HBM
//     into operand registers (128-bit loads), Q^T resident in registers.
//   Online softmax on S^T columns in the log2 domain (scale and sink pre-multiplied by log2 e).
//   O^T (64 d x 16 heads) += V^T (64 x 64) . P^T (64 x 16): 8 MFMA 16x16x32. P^T comes straight
//     from the S^T accumulator registers (same lanes, same columns); V goes row-major into a
//     wave-private LDS tile (128-bit writes) and comes back transposed through the gfx950
//     transpose read, so no element-wise transposition is needed.

#include "chunk_merge.h"
#include "device_common.h"
#include "launch.h"

namespace sinkattn {
namespace {

constexpr int kSplitWaves = 4;
constexpr int kSplitThreads = kSplitWaves * 64;
constexpr int kBlockKeys = 64;  // keys per wave iteration
// V tile row pitch in bf16 elements: 64 + 16 pad = 160 bytes = 40 dwords. The transpose reads of
// 8 consecutive rows then start on 8 disjoint 8-bank groups (conflict-free per half-wave).
constexpr int kVPitch = 80;

// One wave's share of a 64-key block: lane (col, grp) holds key rows base + 16t + col (t = 0..3),
// 16-byte segments grp and grp + 4 of each row, for K and for V.
struct KvBlock {
    bf16x8 k[4][2];
    bf16x8 v[4][2];
};

// Keys at or past the chunk end fall outside the buffer ranges and load as zeros.
__device__ __forceinline__ void load_block(KvBlock& r, __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                           uint32_t k_row_bytes, uint32_t v_row_bytes, uint32_t base,
                                           int col, int grp) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t key = base + 16 * t + col;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t off = 16 * (grp + 4 * h);
            r.k[t][h] = buffer_load_x8(krs, key * k_row_bytes + off);
            r.v[t][h] = buffer_load_x8(vrs, key * v_row_bytes + off);
        }
    }
}

struct SplitState {
    f32x4 acc[4];  // O^T block n: rows d = 16n + 4grp + i, column = head col
    float m;       // running max, log2 units (uniform over the column's four lanes)
    float dsum;    // this lane's share of the running scale d
};

// Folds one 64-key block into the wave's state.
//   S^T (64 x 16) = K . Q^T with K straight from registers;
//   P^T k-slots for key group u (32 keys): slots 0..3 = keys 32u + 4grp + e (S^T block 2u),
//   slots 4..7 = keys 32u + 16 + 4grp + e (S^T block 2u + 1), which is where this lane's S^T
//   values already sit; V^T operands come from the wave's row-major V tile via transpose reads.
__device__ __forceinline__ void fold_block(SplitState& st, const KvBlock& r, const bf16x8 (&q_op)[2],
                                           __bf16 (*vl)[kVPitch], int base, int hi,
                                           float c2, int col, int grp) {
    lds_order();
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            *reinterpret_cast<bf16x8*>(&vl[16 * t + col][8 * (grp + 4 * h)]) = r.v[t][h];

    f32x4 s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        s[t] = mfma16x16x32(r.k[t][0], q_op[0], zero_f32x4());
        s[t] = mfma16x16x32(r.k[t][1], q_op[1], s[t]);
    }
    const bool tail = base + kBlockKeys > hi;
    float x[16];
    float bmax = kNegInf;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v = s[t][i] * c2;
            if (tail && base + 16 * t + 4 * grp + i >= hi) v = kNegInf;
            x[4 * t + i] = v;
            bmax = fmaxf(bmax, v);
        }
    bmax = max_over_groups(bmax);
    const float m_new = fmaxf(st.m, bmax);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = exp2_fast(st.m - m_use);
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        x[e] = exp2_fast(x[e] - m_use);
        psum += x[e];
    }
    st.dsum = st.dsum * alpha + psum;
    st.m = m_new;
#pragma unroll
    for (int n = 0; n < 4; ++n) st.acc[n] *= alpha;

    bf16x8 p_op[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p_op[u][e] = (__bf16)x[4 * (2 * u) + e];
            p_op[u][4 + e] = (__bf16)x[4 * (2 * u + 1) + e];
        }

    lds_order();
    // Transpose-read addressing: lane (grp, col) points at row 4grp + col/4 (+16 for slots 4..7)
    // and columns 16n + 4(col%4); it receives column 16n + col of rows 4grp + 0..3.
    const int tr_row = 4 * grp + (col >> 2);
    const int tr_col = 4 * (col & 3);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const bf16x4 lo4 = lds_read_tr4(&vl[32 * u + tr_row][16 * n + tr_col]);
            const bf16x4 hi4 = lds_read_tr4(&vl[32 * u + 16 + tr_row][16 * n + tr_col]);
            const bf16x8 v_op = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            st.acc[n] = mfma16x16x32(v_op, p_op[u], st.acc[n]);
        }
    lds_order();
}

// kHeads KV heads per work-group, four waves each. With two, the work-group reads both
// heads' 128-byte slices of every cache row together (256 contiguous bytes of a token-major
// row), which the memory system serves measurably faster than lone 128-byte slices.
template <int kHeads, bool kFused>
__global__ __launch_bounds__(kSplitThreads * kHeads) void decode_split_bf16_kernel(DecodeSplitParams p) {
    constexpr int kWaves = kSplitWaves * kHeads;
    __shared__ int last_arrival;
    __shared__ __attribute__((aligned(16))) __bf16 v_tile[kWaves][kBlockKeys][kVPitch];
    __shared__ __attribute__((aligned(16))) float red_m[kWaves][16];
    __shared__ __attribute__((aligned(16))) float red_d[kWaves][16];
    __shared__ __attribute__((aligned(16))) float red_o[kWaves][16][kHeadDim + 4];

    const int lane = threadIdx.x & 63;
    // Wave index in an SGPR: the block loop below is then wave-uniform control flow.
    const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hsub = wave_all / kSplitWaves;  // which of the work-group's KV heads
    const int wave = wave_all % kSplitWaves;  // wave within that head's team
    const int col = lane & 15;  // MFMA column: query head within the group
    const int grp = lane >> 4;  // k-slot group / row quad

    // KV head fastest: the work-groups that read the Hkv interleaved 128-byte slices of the same
    // cache rows are dispatched together.
    int bid = blockIdx.x;
    const int heads_per_row = p.num_kv_heads / kHeads;
    const int head_set = bid % heads_per_row;  // this work-group's KV heads: kHeads * head_set + ...
    const int g = head_set * kHeads + hsub;
    bid /= heads_per_row;
    const int chunk = bid % p.num_chunks;
    const int b = bid / p.num_chunks;
    const int group = p.num_q_heads / p.num_kv_heads;
    const bool col_valid = col < group;
    const int head = g * group + (col_valid ? col : 0);

    int len = p.seqlens_k[b];
    len = len < 0 ? 0 : (len > p.capacity ? static_cast<int>(p.capacity) : len);
    const int64_t lo = static_cast<int64_t>(chunk) * p.chunk_size;
    const int64_t hi = lo + p.chunk_size < len ? lo + p.chunk_size : len;

    const __bf16* qbase = static_cast<const __bf16*>(p.q) + b * p.q_stride_b + head * p.q_stride_head;
    bf16x8 q_op[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        q_op[h] = col_valid ? *reinterpret_cast<const bf16x8*>(qbase + 32 * h + 8 * grp) : zero_bf16x8();

    const float c2 = p.scale * kLog2e;
    SplitState st;
    st.m = kNegInf;
    st.dsum = 0.0f;
    if (chunk == 0 && wave == 0) {
        // The first chunk starts from the sink: m = sink (log2 units), d = 1 = e^(sink - sink).
        st.m = p.sinks[head] * kLog2e;
        st.dsum = (grp == 0 && st.m != kNegInf) ? 1.0f : 0.0f;
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) st.acc[n] = zero_f32x4();

    // Buffer ranges end at the chunk end: rows [0, hi) of this (sequence, KV head) slice.
    const __bf16* kbase = static_cast<const __bf16*>(p.k) + b * p.k_stride_b + g * p.k_stride_head;
    const __bf16* vbase = static_cast<const __bf16*>(p.v) + b * p.v_stride_b + g * p.v_stride_head;
    const uint32_t k_row_bytes = static_cast<uint32_t>(p.k_stride_tok * 2);
    const uint32_t v_row_bytes = static_cast<uint32_t>(p.v_stride_tok * 2);
    const __amdgpu_buffer_rsrc_t krs = make_buffer(kbase, static_cast<uint32_t>(hi) * k_row_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_buffer(vbase, static_cast<uint32_t>(hi) * v_row_bytes);
    __bf16(*vl)[kVPitch] = v_tile[wave_all];

    // Blocks of this wave: base = lo + 64 * (wave + 4 i). Two register sets alternate so the next
    // block's 16 loads per lane are in flight while the current block is folded. The prefetch is
    // unconditional: past the chunk end it returns zeros without touching memory.
    constexpr uint32_t kStride = kSplitWaves * kBlockKeys;
    uint32_t base = static_cast<uint32_t>(lo) + wave * kBlockKeys;
    const uint32_t end = static_cast<uint32_t>(hi);
    // The scheduling barriers keep each prefetch ahead of the math that waits on the previous
    // block, so two blocks' loads are in flight at every wait.
    KvBlock ra, rb;
    load_block(ra, krs, vrs, k_row_bytes, v_row_bytes, base, col, grp);
    while (base < end) {
        load_block(rb, krs, vrs, k_row_bytes, v_row_bytes, base + kStride, col, grp);
        __builtin_amdgcn_sched_barrier(0);
        fold_block(st, ra, q_op, vl, static_cast<int>(base), static_cast<int>(hi), c2, col, grp);
        base += kStride;
        if (base >= end) break;
        load_block(ra, krs, vrs, k_row_bytes, v_row_bytes, base + kStride, col, grp);
        __builtin_amdgcn_sched_barrier(0);
        fold_block(st, rb, q_op, vl, static_cast<int>(base), static_cast<int>(hi), c2, col, grp);
        base += kStride;
    }

    // Merge each head's four wave states (log2 domain) and write the chunk's (m, d, o).
    const float d_wave = sum_over_groups(st.dsum);
    if (grp == 0) {
        red_m[wave_all][col] = st.m;
        red_d[wave_all][col] = d_wave;
    }
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) red_o[wave_all][col][16 * n + 4 * grp + i] = st.acc[n][i];
    __syncthreads();

    const int team_tid = threadIdx.x % kSplitThreads;
    const int w0 = hsub * kSplitWaves;
    for (int idx = team_tid; idx < group * kHeadDim; idx += kSplitThreads) {
        const int hc = idx / kHeadDim;
        const int d = idx % kHeadDim;
        float big = kNegInf;
#pragma unroll
        for (int w = 0; w < kSplitWaves; ++w) big = fmaxf(big, red_m[w0 + w][hc]);
        float wsum = 0.0f, osum = 0.0f;
        if (big != kNegInf) {
#pragma unroll
            for (int w = 0; w < kSplitWaves; ++w) {
                const float f = exp2_fast(red_m[w0 + w][hc] - big);
                wsum += red_d[w0 + w][hc] * f;
                osum += red_o[w0 + w][hc][d] * f;
            }
        }
        const int64_t row = (static_cast<int64_t>(b) * p.num_q_heads + g * group + hc) * p.num_chunks + chunk;
        const float o = wsum > 0.0f ? osum / wsum : 0.0f;
        const float m_nat = wsum > 0.0f ? big * kLn2 : kNegInf;
        if constexpr (kFused) {
            // Write-through stores: the release fence below then has no dirty L2 lines to write
            // back, which is most of its cost (38 -> 34 us on 8 x 8192 keys).
            __hip_atomic_store(&p.partial_o[row * kHeadDim + d], o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            if (d == 0) {
                __hip_atomic_store(&p.partial_m[row], m_nat, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                __hip_atomic_store(&p.partial_d[row], wsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            }
        } else {
            p.partial_o[row * kHeadDim + d] = o;
            if (d == 0) {
                p.partial_m[row] = m_nat;
                p.partial_d[row] = wsum;
            }
        }
    }

    if constexpr (kFused) {
        // Publish this chunk's states, then count the work-group done for its (sequence, KV
        // heads). The barrier orders every wave's stores before thread 0's device-scope release
        // fence (an L2 write-back); only the last arrival takes the acquire fence (an L2 and L1
        // invalidate), after which it reads every chunk's states whichever XCD produced them.
        __syncthreads();
        uint32_t* counter = p.counters + static_cast<int64_t>(b) * heads_per_row + head_set;
        if (threadIdx.x == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            const bool last = atomicAdd(counter, 1u) == static_cast<uint32_t>(p.num_chunks - 1);
            if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            last_arrival = last;
        }
        __syncthreads();
        if (!last_arrival) return;
        // Log-sum-exp merge of all chunks for this work-group's kHeads * G query heads, one wave
        // per head at a time.
        const int lane = threadIdx.x & 63;
        for (int hl = wave_all; hl < kHeads * group; hl += kWaves) {
            const int h = head_set * kHeads * group + hl;
            const int64_t bh = static_cast<int64_t>(b) * p.num_q_heads + h;
            float o, lse;
            merge_chunk_states(p.partial_m + bh * p.num_chunks, p.partial_d + bh * p.num_chunks,
                               p.partial_o + bh * p.num_chunks * kHeadDim, p.num_chunks, lane, o, lse);
            const int64_t off = b * p.o_stride_b + h * p.o_stride_head + lane;
            if (p.out_is_bf16)
                static_cast<__bf16*>(p.out)[off] = (__bf16)o;
            else
                static_cast<float*>(p.out)[off] = o;
            if (p.lse != nullptr && lane == 0) p.lse[b * p.lse_stride_b + h * p.lse_stride_head] = lse;
        }
        // Leave the counter at zero for the next call.
        if (threadIdx.x == 0) atomicExch(counter, 0u);
    }
}

// fp32 reference variant: one thread per (b, query head, chunk), keys visited one at a time with
// the page's online recurrence (tile of one key). Written for clarity, not speed.
__global__ __launch_bounds__(256) void decode_split_f32_kernel(DecodeSplitParams p) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = static_cast<int64_t>(p.batch) * p.num_q_heads * p.num_chunks;
    if (idx >= total) return;
    const int chunk = static_cast<int>(idx % p.num_chunks);
    const int head = static_cast<int>((idx / p.num_chunks) % p.num_q_heads);
    const int b = static_cast<int>(idx / (static_cast<int64_t>(p.num_chunks) * p.num_q_heads));
    const int g = head / (p.num_q_heads / p.num_kv_heads);

    int len = p.seqlens_k[b];
    len = len < 0 ? 0 : (len > p.capacity ? static_cast<int>(p.capacity) : len);
    const int64_t lo = static_cast<int64_t>(chunk) * p.chunk_size;
    const int64_t hi = lo + p.chunk_size < len ? lo + p.chunk_size : len;

    const float* qrow = static_cast<const float*>(p.q) + b * p.q_stride_b + head * p.q_stride_head;
    float qv[kHeadDim], acc[kHeadDim];
    for (int d = 0; d < kHeadDim; ++d) {
        qv[d] = qrow[d];
        acc[d] = 0.0f;
    }
    float m = kNegInf, dsum = 0.0f;
    if (chunk == 0) {
        m = p.sinks[head];
        dsum = m == kNegInf ? 0.0f : 1.0f;
    }
    const float* kb = static_cast<const float*>(p.k) + b * p.k_stride_b + g * p.k_stride_head;
    const float* vb = static_cast<const float*>(p.v) + b * p.v_stride_b + g * p.v_stride_head;
    for (int64_t j = lo; j < hi; ++j) {
        const float* kr = kb + j * p.k_stride_tok;
        const float* vr = vb + j * p.v_stride_tok;
        float s = 0.0f;
        for (int d = 0; d < kHeadDim; ++d) s = fmaf(qv[d], kr[d], s);
        s *= p.scale;
        if (s > m) {
            const float alpha = m == kNegInf ? 0.0f : expf(m - s);
            dsum = dsum * alpha + 1.0f;
            for (int d = 0; d < kHeadDim; ++d) acc[d] = acc[d] * alpha + vr[d];
            m = s;
        } else {
            const float pj = expf(s - m);
            dsum += pj;
            for (int d = 0; d < kHeadDim; ++d) acc[d] = fmaf(pj, vr[d], acc[d]);
        }
    }
    const int64_t row = idx;  // (b, head, chunk) row-major == idx
    const float inv = dsum > 0.0f ? 1.0f / dsum : 0.0f;
    for (int d = 0; d < kHeadDim; ++d) p.partial_o[row * kHeadDim + d] = acc[d] * inv;
    p.partial_m[row] = dsum > 0.0f ? m : kNegInf;
    p.partial_d[row] = dsum;
}

}  // namespace

// Compute units of an MI355X / MI350X (gfx950).
constexpr int64_t kComputeUnits = 256;

template <bool kFused>
hipError_t launch_split(const DecodeSplitParams& p, hipStream_t stream) {
    // Pair two KV heads per work-group only where their slices of a cache row are adjacent
    // (token-major caches) and the paired grid still gives every compute unit a work-group;
    // head-major caches already stream contiguous rows and prefer the finer grid.
    const bool adjacent = p.k_stride_head == kHeadDim && p.v_stride_head == kHeadDim;
    const int64_t paired_groups = static_cast<int64_t>(p.batch) * (p.num_kv_heads / 2) * p.num_chunks;
    if (p.num_kv_heads % 2 == 0 && adjacent && paired_groups >= kComputeUnits) {
        decode_split_bf16_kernel<2, kFused>
            <<<dim3(static_cast<unsigned>(paired_groups)), dim3(2 * kSplitThreads), 0, stream>>>(p);
    } else {
        const int64_t blocks = static_cast<int64_t>(p.batch) * p.num_kv_heads * p.num_chunks;
        decode_split_bf16_kernel<1, kFused>
            <<<dim3(static_cast<unsigned>(blocks)), dim3(kSplitThreads), 0, stream>>>(p);
    }
    return hipGetLastError();
}

hipError_t launch_decode_split_bf16(const DecodeSplitParams& p, hipStream_t stream) {
    return launch_split<false>(p, stream);
}

hipError_t launch_decode_fused_bf16(const DecodeSplitParams& p, hipStream_t stream) {
    return launch_split<true>(p, stream);
}

hipError_t launch_decode_split_f32(const DecodeSplitParams& p, hipStream_t stream) {
    const int64_t total = static_cast<int64_t>(p.batch) * p.num_q_heads * p.num_chunks;
    const int64_t blocks = (total + 255) / 256;
    decode_split_f32_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace sinkattn
