// Causal varlen prefill with a learned per-head softmax sink (gfx950).
//
// Source: "GPT-OSS on Day 0" (Perplexity), section "Kernels for GPT-OSS", subsection "Sink
// attention": softmax over the scaled Q.K^T scores extended by the head's sink logit, evaluated
// online with a running max m started at the sink value and a running scale d started at 1. One
// work-group walks every KV tile of its rows, so the sink is folded once per row, before the
// first tile (the "first chunk" of that subsection).
//
// bf16 path. One work-group = (query tile, KV head g). Its 128 query rows are
// (128 / G) consecutive positions x the G query heads that share KV head g (heads fastest), so
// every K/V tile staged in LDS serves G times as many rows as an MHA tile would, and the causal
// diagonal is only 128 / G positions wide. Four waves own 32 rows each (two 16-column MFMA blocks).
// Per 64-key tile, per wave:
//   S^T (64 keys x 32 rows) = K (LDS, row-major) . Q^T (registers): 16 MFMA 16x16x32 bf16.
//   online softmax per row (log2 domain; scale and sink pre-multiplied by log2 e), causal mask
//     only on tiles that cross the diagonal or the sequence end.
//   O^T (64 d x 32 rows) += V^T (LDS, stored transposed) . P^T (registers): 16 MFMA. The S^T
//     accumulator lanes are exactly the P^T operand lanes, so P never leaves registers.
// The next tile's K/V global loads are issued before the current tile's math.
// Work-groups are numbered query-tile-major with the KV head fastest, so consecutive
// work-groups (which the dispatcher spreads over the eight XCDs) read different KV heads and each
// XCD's L2 keeps re-serving one head's K/V. Within a sequence, tiles are issued last-position
// first: the longest causal rows start earliest.

#include "device_common.h"
#include "launch.h"

namespace sinkattn {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerTile = kPfWaves * kRowsPerWave;  // 128
constexpr int kKeyTile = 64;
constexpr int kKPitch = 72;   // K tile row: 64 + 8 pad bf16 = 144 B; conflict-free 16 B operand reads
constexpr int kVtPitch = 68;  // V^T tile row: 64 + 4 pad bf16 = 136 B; 8 B operand reads

// Maps a linear query-tile index to (sequence, first position). Tiles are numbered sequence by
// sequence; within a sequence index 0 is the tile holding the last positions. Returns false for
// the padding tiles past the last one.
__device__ bool locate_tile(const int32_t* cu_q, int num_seqs, int total_q, int positions_per_tile,
                            int tile, int& seq, int& first_pos, int& q_start, int& q_len) {
    int before = 0;
    for (int s = 0; s < num_seqs; ++s) {
        // Clamped so that malformed prefix sums cannot move a row outside [0, total_q).
        const int start = min(max(cu_q[s], 0), total_q);
        const int len = min(max(cu_q[s + 1] - start, 0), total_q - start);
        const int tiles = (len + positions_per_tile - 1) / positions_per_tile;
        if (tile < before + tiles) {
            seq = s;
            first_pos = (tiles - 1 - (tile - before)) * positions_per_tile;
            q_start = start;
            q_len = len;
            return true;
        }
        before += tiles;
    }
    return false;
}

__global__ __launch_bounds__(kPfThreads, 2) void prefill_bf16_kernel(PrefillParams p) {
    __shared__ __attribute__((aligned(16))) __bf16 k_tile[kKeyTile][kKPitch];
    __shared__ __attribute__((aligned(16))) __bf16 vt_tile[kHeadDim][kVtPitch];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;
    const int grp = lane >> 4;

    const int g = blockIdx.x % p.num_kv_heads;
    const int tile = blockIdx.x / p.num_kv_heads;
    const int group = p.num_q_heads / p.num_kv_heads;
    const int positions_per_tile = kRowsPerTile / group;

    int seq, first_pos, q_start, q_len;
    if (!locate_tile(p.cu_seqlens_q, p.num_seqs, static_cast<int>(p.total_q), positions_per_tile, tile,
                     seq, first_pos, q_start, q_len))
        return;
    const int total_k = static_cast<int>(p.total_k);
    const int k_start = min(max(p.cu_seqlens_k[seq], 0), total_k);
    const int k_len = min(max(p.cu_seqlens_k[seq + 1] - k_start, 0), total_k - k_start);
    const int offset = k_len - q_len;  // bottom-right causal alignment

    // Rows of this lane: column block cb -> tile row wave*32 + cb*16 + col.
    int pos[2], head[2];
    bool valid[2];
    const float c2 = p.scale * kLog2e;
    bf16x8 q_op[2][2];
    float m[2], dsum[2];
    f32x4 acc[2][4];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int r = wave * kRowsPerWave + cb * 16 + col;
        pos[cb] = first_pos + r / group;
        head[cb] = g * group + r % group;
        valid[cb] = pos[cb] < q_len;
        const __bf16* qrow = static_cast<const __bf16*>(p.q) +
                             static_cast<int64_t>(q_start + pos[cb]) * p.q_stride_tok +
                             static_cast<int64_t>(head[cb]) * p.q_stride_head;
#pragma unroll
        for (int h = 0; h < 2; ++h)
            q_op[cb][h] = valid[cb] ? *reinterpret_cast<const bf16x8*>(qrow + 32 * h + 8 * grp) : zero_bf16x8();
        // Sink fold: m starts at the head's sink, d at 1 (kept in the grp-0 lane's partial sum).
        m[cb] = p.sinks[head[cb]] * kLog2e;
        dsum[cb] = (grp == 0 && m[cb] != kNegInf) ? 1.0f : 0.0f;
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[cb][n] = zero_f32x4();
    }

    // Keys this tile's rows may see: [0, key_end).
    const int last_pos = min(first_pos + positions_per_tile, q_len) - 1;
    int key_end = p.causal ? min(k_len, last_pos + offset + 1) : k_len;
    key_end = key_end < 0 ? 0 : key_end;
    // Tiles at or past this key index need masking (diagonal or sequence end).
    const int safe_end = p.causal ? min(k_len, first_pos + offset + 1) : k_len;
    const int num_tiles = (key_end + kKeyTile - 1) / kKeyTile;

    const __bf16* kbase = static_cast<const __bf16*>(p.k) + static_cast<int64_t>(k_start) * p.k_stride_tok +
                          static_cast<int64_t>(g) * p.k_stride_head;
    const __bf16* vbase = static_cast<const __bf16*>(p.v) + static_cast<int64_t>(k_start) * p.v_stride_tok +
                          static_cast<int64_t>(g) * p.v_stride_head;

    // Global->register staging. K: thread owns rows tid/8 and tid/8 + 32, segment tid%8 (full
    // 128-byte rows per 8 lanes). V: row (lane%16) + 16*wave, segments lane/16 and lane/16 + 4.
    const int k_row = tid >> 3, k_seg = tid & 7;
    const int v_row = (lane & 15) + 16 * wave, v_seg = lane >> 4;
    bf16x8 kst[2], vst[2];
    auto fetch = [&](int key0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int kr = key0 + k_row + 32 * i;
            kst[i] = kr < key_end ? *reinterpret_cast<const bf16x8*>(kbase + static_cast<int64_t>(kr) * p.k_stride_tok + 8 * k_seg)
                                  : zero_bf16x8();
            const int vr = key0 + v_row;
            vst[i] = vr < key_end ? *reinterpret_cast<const bf16x8*>(vbase + static_cast<int64_t>(vr) * p.v_stride_tok + 8 * (v_seg + 4 * i))
                                  : zero_bf16x8();
        }
    };

    if (num_tiles > 0) fetch(0);
    for (int kt = 0; kt < num_tiles; ++kt) {
        const int key0 = kt * kKeyTile;
        __syncthreads();  // previous tile fully consumed
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            *reinterpret_cast<bf16x8*>(&k_tile[k_row + 32 * i][8 * k_seg]) = kst[i];
#pragma unroll
            for (int e = 0; e < 8; ++e) vt_tile[8 * (v_seg + 4 * i) + e][v_row] = vst[i][e];
        }
        __syncthreads();
        if (kt + 1 < num_tiles) fetch(key0 + kKeyTile);

        // S^T: block t holds keys key0 + 16t + 4grp + i (rows), query rows (columns).
        f32x4 s[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bf16x8 ka0 = *reinterpret_cast<const bf16x8*>(&k_tile[16 * t + col][8 * grp]);
            const bf16x8 ka1 = *reinterpret_cast<const bf16x8*>(&k_tile[16 * t + col][32 + 8 * grp]);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                s[t][cb] = mfma16x16x32(ka0, q_op[cb][0], zero_f32x4());
                s[t][cb] = mfma16x16x32(ka1, q_op[cb][1], s[t][cb]);
            }
        }

        const bool need_mask = key0 + kKeyTile > safe_end;
        bf16x8 p_op[2][2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            float x[16];
            float bmax = kNegInf;
            const int limit = p.causal ? min(k_len, pos[cb] + offset + 1) : k_len;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = s[t][cb][i] * c2;
                    if (need_mask && key0 + 16 * t + 4 * grp + i >= limit) v = kNegInf;
                    x[4 * t + i] = v;
                    bmax = fmaxf(bmax, v);
                }
            bmax = max_over_groups(bmax);
            const float m_new = fmaxf(m[cb], bmax);
            const float m_use = m_new == kNegInf ? 0.0f : m_new;
            const float alpha = exp2_fast(m[cb] - m_use);
            float psum = 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                x[e] = exp2_fast(x[e] - m_use);
                psum += x[e];
            }
            dsum[cb] = dsum[cb] * alpha + psum;
            m[cb] = m_new;
#pragma unroll
            for (int n = 0; n < 4; ++n) acc[cb][n] *= alpha;
            // P^T operand for key group u: slots 0..3 = block 2u, slots 4..7 = block 2u + 1.
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    p_op[cb][u][e] = (__bf16)x[4 * (2 * u) + e];
                    p_op[cb][u][4 + e] = (__bf16)x[4 * (2 * u + 1) + e];
                }
        }

        // O^T += V^T . P^T. V^T operand rows d = 16n + col; k-slots as in p_op.
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const __bf16* row = &vt_tile[16 * n + col][32 * u];
                const bf16x4 lo4 = *reinterpret_cast<const bf16x4*>(row + 4 * grp);
                const bf16x4 hi4 = *reinterpret_cast<const bf16x4*>(row + 16 + 4 * grp);
                const bf16x8 v_op = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) acc[cb][n] = mfma16x16x32(v_op, p_op[cb][u], acc[cb][n]);
            }
    }

    // Epilogue: out = acc / d. Lane holds d-channels 16n + 4grp + i of its rows.
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const float dtot = sum_over_groups(dsum[cb]);
        if (!valid[cb]) continue;
        const float inv = dtot > 0.0f ? 1.0f / dtot : 0.0f;
        const int64_t obase = static_cast<int64_t>(q_start + pos[cb]) * p.o_stride_tok +
                              static_cast<int64_t>(head[cb]) * p.o_stride_head;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int d0 = 16 * n + 4 * grp;
            if (p.out_is_bf16) {
                bf16x4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = (__bf16)(acc[cb][n][i] * inv);
                *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.out) + obase + d0) = o;
            } else {
                *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + obase + d0) = acc[cb][n] * inv;
            }
        }
    }
}

// fp32 reference variant: one thread per (query head, token); keys visited one at a time with
// the page's online recurrence. Lanes of a wave are consecutive tokens of one head, so they read
// the same key rows. Written for clarity, not speed.
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillParams p) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= p.total_q * p.num_q_heads) return;
    const int head = static_cast<int>(idx / p.total_q);
    const int tok = static_cast<int>(idx % p.total_q);
    const int g = head / (p.num_q_heads / p.num_kv_heads);

    // Sequence of this token: last s with cu_q[s] <= tok (binary search over B+1 prefix sums).
    int lo = 0, hi = p.num_seqs;  // answer in [lo, hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.cu_seqlens_q[mid] <= tok) lo = mid; else hi = mid;
    }
    const int seq = lo;
    // Clamped so that malformed prefix sums cannot move a key row outside [0, total_k).
    const int total_k = static_cast<int>(p.total_k);
    const int q_start = p.cu_seqlens_q[seq];
    const int q_len = p.cu_seqlens_q[seq + 1] - q_start;
    const int k_start = min(max(p.cu_seqlens_k[seq], 0), total_k);
    const int k_len = min(max(p.cu_seqlens_k[seq + 1] - k_start, 0), total_k - k_start);
    const int i = tok - q_start;
    int key_end = p.causal ? min(k_len, i + (k_len - q_len) + 1) : k_len;
    key_end = key_end < 0 ? 0 : key_end;

    const float* qrow = static_cast<const float*>(p.q) + static_cast<int64_t>(tok) * p.q_stride_tok +
                        static_cast<int64_t>(head) * p.q_stride_head;
    float qv[kHeadDim], acc[kHeadDim];
    for (int d = 0; d < kHeadDim; ++d) {
        qv[d] = qrow[d];
        acc[d] = 0.0f;
    }
    float m = p.sinks[head];
    float dsum = m == kNegInf ? 0.0f : 1.0f;
    const float* kb = static_cast<const float*>(p.k) + static_cast<int64_t>(k_start) * p.k_stride_tok +
                      static_cast<int64_t>(g) * p.k_stride_head;
    const float* vb = static_cast<const float*>(p.v) + static_cast<int64_t>(k_start) * p.v_stride_tok +
                      static_cast<int64_t>(g) * p.v_stride_head;
    for (int j = 0; j < key_end; ++j) {
        const float* kr = kb + static_cast<int64_t>(j) * p.k_stride_tok;
        const float* vr = vb + static_cast<int64_t>(j) * p.v_stride_tok;
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
    const float inv = dsum > 0.0f ? 1.0f / dsum : 0.0f;
    float* orow = static_cast<float*>(p.out) + static_cast<int64_t>(tok) * p.o_stride_tok +
                  static_cast<int64_t>(head) * p.o_stride_head;
    for (int d = 0; d < kHeadDim; ++d) orow[d] = acc[d] * inv;
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream) {
    const int group = p.num_q_heads / p.num_kv_heads;
    const int positions_per_tile = kRowsPerTile / group;
    // Upper bound on query tiles without reading cu_seqlens: each sequence adds at most one
    // partial tile beyond ceil(Tq / positions_per_tile).
    const int64_t tiles = (p.total_q + positions_per_tile - 1) / positions_per_tile + p.num_seqs;
    const int64_t blocks = tiles * p.num_kv_heads;
    if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
    prefill_bf16_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(kPfThreads), 0, stream>>>(p);
    return hipGetLastError();
}

hipError_t launch_prefill_f32(const PrefillParams& p, hipStream_t stream) {
    const int64_t total = p.total_q * p.num_q_heads;
    const int64_t blocks = (total + 255) / 256;
    if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
    prefill_f32_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace sinkattn
