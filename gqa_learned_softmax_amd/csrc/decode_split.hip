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
// Per 32-key block, per wave:
//   S^T (32 keys x 16 heads) = K (32 x 64) . Q^T (64 x 16): 4 MFMA 16x16x32, K straight from HBM
//     (128-bit loads, 16 lanes x 16 bytes cover a key row segment), Q^T resident in registers.
//   Online softmax on S^T columns in the log2 domain (scale and sink pre-multiplied by log2 e).
//   O^T (64 d x 16 heads) += V^T (64 x 32) . P^T (32 x 16): 4 MFMA 16x16x32. P^T comes straight
//     from the S^T accumulator registers (same lanes, same columns); V^T is staged through a
//     wave-private LDS tile, written transposed.

#include "device_common.h"
#include "launch.h"

namespace sinkattn {
namespace {

constexpr int kSplitWaves = 4;
constexpr int kSplitThreads = kSplitWaves * 64;
constexpr int kKeysPerBlock = 32;
// V^T tile row pitch in bf16 elements: 32 keys + 8 pad (80 bytes = 20 dwords). Rows stay 8-byte
// aligned for the 64-bit operand reads, which then hit 64 distinct banks per 32 lanes; the
// transposed 2-byte writes see at most 2-way bank conflicts.
constexpr int kVtPitch = 40;

__global__ __launch_bounds__(kSplitThreads) void decode_split_bf16_kernel(DecodeSplitParams p) {
    __shared__ __attribute__((aligned(16))) __bf16 vt_tile[kSplitWaves][kHeadDim][kVtPitch];
    __shared__ __attribute__((aligned(16))) float red_m[kSplitWaves][16];
    __shared__ __attribute__((aligned(16))) float red_d[kSplitWaves][16];
    __shared__ __attribute__((aligned(16))) float red_o[kSplitWaves][16][kHeadDim + 4];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;  // MFMA column: query head within the group
    const int grp = lane >> 4;  // k-slot group / row quad

    int bid = blockIdx.x;
    const int chunk = bid % p.num_chunks;
    bid /= p.num_chunks;
    const int g = bid % p.num_kv_heads;
    const int b = bid / p.num_kv_heads;
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
    float m = kNegInf;
    float dsum = 0.0f;
    if (chunk == 0 && wave == 0) {
        // The first chunk starts from the sink: m = sink (log2 units), d = 1 = e^(sink - sink).
        m = p.sinks[head] * kLog2e;
        dsum = (grp == 0 && m != kNegInf) ? 1.0f : 0.0f;
    }
    f32x4 acc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[n] = zero_f32x4();

    const __bf16* kbase = static_cast<const __bf16*>(p.k) + b * p.k_stride_b + g * p.k_stride_head;
    const __bf16* vbase = static_cast<const __bf16*>(p.v) + b * p.v_stride_b + g * p.v_stride_head;
    __bf16(*vt)[kVtPitch] = vt_tile[wave];

    for (int64_t base = lo + wave * kKeysPerBlock; base < hi; base += kSplitWaves * kKeysPerBlock) {
        // Lane (col, grp) owns key rows base + 16t + col (t = 0, 1) and the 16-byte segments
        // grp and grp + 4 of each row.
        bf16x8 kreg[2][2], vreg[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int64_t key = base + 16 * t + col;
            const bool ok = key < hi;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int off = 8 * (grp + 4 * h);
                kreg[t][h] = ok ? *reinterpret_cast<const bf16x8*>(kbase + key * p.k_stride_tok + off)
                                : zero_bf16x8();
                vreg[t][h] = ok ? *reinterpret_cast<const bf16x8*>(vbase + key * p.v_stride_tok + off)
                                : zero_bf16x8();
            }
        }
        // V^T into the wave's LDS tile: element (key 16t + col, d = 8*(grp + 4h) + e).
        lds_order();
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) vt[8 * (grp + 4 * h) + e][16 * t + col] = vreg[t][h][e];

        // S^T blocks: rows = keys base + 16t + 4grp + i, column = head col.
        f32x4 s[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            s[t] = mfma16x16x32(kreg[t][0], q_op[0], zero_f32x4());
            s[t] = mfma16x16x32(kreg[t][1], q_op[1], s[t]);
        }
        float x[8];
        float bmax = kNegInf;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t key = base + 16 * t + 4 * grp + i;
                const float v = key < hi ? s[t][i] * c2 : kNegInf;
                x[4 * t + i] = v;
                bmax = fmaxf(bmax, v);
            }
        bmax = max_over_groups(bmax);
        const float m_new = fmaxf(m, bmax);
        const float m_use = m_new == kNegInf ? 0.0f : m_new;
        const float alpha = exp2_fast(m - m_use);
        float psum = 0.0f;
        bf16x8 p_op;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pe = exp2_fast(x[e] - m_use);
            psum += pe;
            p_op[e] = (__bf16)pe;
        }
        dsum = dsum * alpha + psum;
        m = m_new;
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[n] *= alpha;

        lds_order();
        // O^T block n: rows d = 16n + col; k-slots e < 4 are keys 4grp + e, e >= 4 are keys
        // 16 + 4grp + (e - 4): exactly the keys whose P values this lane holds.
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const __bf16* row = vt[16 * n + col];
            bf16x4 lo4 = *reinterpret_cast<const bf16x4*>(row + 4 * grp);
            bf16x4 hi4 = *reinterpret_cast<const bf16x4*>(row + 16 + 4 * grp);
            bf16x8 v_op = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            acc[n] = mfma16x16x32(v_op, p_op, acc[n]);
        }
        lds_order();
    }

    // Merge the four waves' states (log2 domain) and write the chunk's (m, d, o).
    const float d_wave = sum_over_groups(dsum);
    if (grp == 0) {
        red_m[wave][col] = m;
        red_d[wave][col] = d_wave;
    }
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) red_o[wave][col][16 * n + 4 * grp + i] = acc[n][i];
    __syncthreads();

    for (int idx = threadIdx.x; idx < group * kHeadDim; idx += kSplitThreads) {
        const int hc = idx / kHeadDim;
        const int d = idx % kHeadDim;
        float big = kNegInf;
#pragma unroll
        for (int w = 0; w < kSplitWaves; ++w) big = fmaxf(big, red_m[w][hc]);
        float wsum = 0.0f, osum = 0.0f;
        if (big != kNegInf) {
#pragma unroll
            for (int w = 0; w < kSplitWaves; ++w) {
                const float f = exp2_fast(red_m[w][hc] - big);
                wsum += red_d[w][hc] * f;
                osum += red_o[w][hc][d] * f;
            }
        }
        const int64_t row = (static_cast<int64_t>(b) * p.num_q_heads + g * group + hc) * p.num_chunks + chunk;
        p.partial_o[row * kHeadDim + d] = wsum > 0.0f ? osum / wsum : 0.0f;
        if (d == 0) {
            p.partial_m[row] = wsum > 0.0f ? big * kLn2 : kNegInf;
            p.partial_d[row] = wsum;
        }
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

hipError_t launch_decode_split_bf16(const DecodeSplitParams& p, hipStream_t stream) {
    const int64_t blocks = static_cast<int64_t>(p.batch) * p.num_kv_heads * p.num_chunks;
    decode_split_bf16_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(kSplitThreads), 0, stream>>>(p);
    return hipGetLastError();
}

hipError_t launch_decode_split_f32(const DecodeSplitParams& p, hipStream_t stream) {
    const int64_t total = static_cast<int64_t>(p.batch) * p.num_q_heads * p.num_chunks;
    const int64_t blocks = (total + 255) / 256;
    decode_split_f32_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace sinkattn
