// Causal varlen prefill with a learned per-head softmax sink (gfx950).
//
// Source: "GPT-OSS on Day 0" (Perplexity), section "Kernels for GPT-OSS", subsection "Sink
// attention": softmax over the scaled Q.K^T scores extended by the head's sink logit, evaluated
// online with a running max m started at the sink value and a running scale d started at 1. One
// work-group walks every KV tile of its rows, so the sink is folded once per row, before the
// first tile (the "first chunk" of that subsection).
//
// bf16 path. One work-group = (query tile, KV head g). Its 256 query rows are (256 / G)
// consecutive positions x the G query heads that share KV head g (heads fastest), so every K/V
// tile staged in LDS serves G times as many rows as an MHA tile would, and the causal diagonal is
// only 256 / G positions wide. Four waves own 64 rows each (two 32-column MFMA blocks).
// Per 64-key tile, per wave (32 v_mfma_f32_32x32x16_bf16, the gfx950 shape with the highest
// sustained rate):
//   S^T (64 keys x 64 rows) = K (LDS, row-major) . Q^T (registers): 16 MFMA.
//   online softmax per row in the log2 domain (scale and sink pre-multiplied by log2 e), one FMA
//     per score for scale-and-subtract, lazy rescaling, causal mask only on tiles that cross
//     the diagonal or the sequence end.
//   O^T (64 d x 64 rows) += V^T . P^T: 16 MFMA. The S^T accumulator lanes are exactly the P^T
//     operand lanes, so P never leaves registers; V stays row-major in LDS and comes back
//     transposed through ds_read_b64_tr_b16.
// K/V tiles are double-buffered in LDS: the next tile's buffer loads are issued before the
// current tile's math and written to the other buffer after it, one barrier per tile.
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
constexpr int kRowsPerWave = 64;                       // two 32-column MFMA blocks
constexpr int kRowsPerTile = kPfWaves * kRowsPerWave;  // 256 query rows per work-group
constexpr int kKeyTile = 64;
// K tile rows: 64 + 8 pad bf16 = 144 B, so 16 consecutive rows start on distinct 4-bank groups
// for the 16-byte operand reads. V tile rows: 64 + 32 pad = 192 B, so the four rows of each
// transpose read land on disjoint bank ranges.
constexpr int kKPitch = 72;
constexpr int kVPitch = 96;
// Lazy rescaling: the running max is only raised (and the accumulators rescaled) when a tile's
// max exceeds it by more than this many log2 units; in between, exp2(s - m) <= 2^8 stays exact
// enough in fp32 and bf16 and the division by d at the end cancels the stale max.
constexpr float kRescaleSlack = 8.0f;

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
    __shared__ __attribute__((aligned(16))) __bf16 k_tile[2][kKeyTile][kKPitch];
    __shared__ __attribute__((aligned(16))) __bf16 v_tile[2][kKeyTile][kVPitch];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;   // MFMA column: query row within a 32-row block
    const int half = lane >> 5;  // k-slot group

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

    // Rows of this lane: column block cb -> tile row 64 wave + 32 cb + col.
    int pos[2], head[2];
    bool valid[2];
    const float c2 = p.scale * kLog2e;
    bf16x8 q_op[2][4];
    float m[2], dsum[2];
    f32x16 acc[2][2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int r = wave * kRowsPerWave + cb * 32 + col;
        pos[cb] = first_pos + r / group;
        head[cb] = g * group + r % group;
        valid[cb] = pos[cb] < q_len;
        const __bf16* qrow = static_cast<const __bf16*>(p.q) +
                             static_cast<int64_t>(q_start + (valid[cb] ? pos[cb] : 0)) * p.q_stride_tok +
                             static_cast<int64_t>(head[cb]) * p.q_stride_head;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            q_op[cb][ks] = valid[cb] ? *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * half) : zero_bf16x8();
        // Sink fold: m starts at the head's sink, d at 1 (kept in the half-0 lane's partial sum).
        m[cb] = p.sinks[head[cb]] * kLog2e;
        dsum[cb] = (half == 0 && m[cb] != kNegInf) ? 1.0f : 0.0f;
#pragma unroll
        for (int n = 0; n < 2; ++n) acc[cb][n] = zero_f32x16();
    }

    // Keys this tile's rows may see: [0, key_end).
    const int last_pos = min(first_pos + positions_per_tile, q_len) - 1;
    int key_end = p.causal ? min(k_len, last_pos + offset + 1) : k_len;
    key_end = key_end < 0 ? 0 : key_end;
    // Tiles reaching past this key need masking (diagonal or sequence end).
    const int safe_end = p.causal ? min(k_len, first_pos + offset + 1) : k_len;
    const int num_tiles = (key_end + kKeyTile - 1) / kKeyTile;

    // K/V rows [0, key_end) of KV head g of this sequence; loads past the end return zeros.
    const __bf16* kbase = static_cast<const __bf16*>(p.k) + static_cast<int64_t>(k_start) * p.k_stride_tok +
                          static_cast<int64_t>(g) * p.k_stride_head;
    const __bf16* vbase = static_cast<const __bf16*>(p.v) + static_cast<int64_t>(k_start) * p.v_stride_tok +
                          static_cast<int64_t>(g) * p.v_stride_head;
    const uint32_t k_row_bytes = static_cast<uint32_t>(p.k_stride_tok * 2);
    const uint32_t v_row_bytes = static_cast<uint32_t>(p.v_stride_tok * 2);
    const __amdgpu_buffer_rsrc_t krs = make_buffer(kbase, static_cast<uint32_t>(key_end) * k_row_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_buffer(vbase, static_cast<uint32_t>(key_end) * v_row_bytes);

    // Staging: thread owns rows tid/8 and tid/8 + 32 of a tile, 16-byte segment tid%8.
    const int ld_row = tid >> 3, ld_seg = tid & 7;
    bf16x8 kst[2], vst[2];
    auto fetch = [&](int key0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t row = static_cast<uint32_t>(key0 + ld_row + 32 * i);
            kst[i] = buffer_load_x8(krs, row * k_row_bytes + 16 * ld_seg);
            vst[i] = buffer_load_x8(vrs, row * v_row_bytes + 16 * ld_seg);
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            *reinterpret_cast<bf16x8*>(&k_tile[buf][ld_row + 32 * i][8 * ld_seg]) = kst[i];
            *reinterpret_cast<bf16x8*>(&v_tile[buf][ld_row + 32 * i][8 * ld_seg]) = vst[i];
        }
    };

    // Transpose-read addressing for the V^T operand (16-lane group a = lane / 16): lane
    // 16a + L points at tile row 4 * (a / 2) + L / 4 (+ 8 for k-slots 4..7) and column
    // 16 * (a % 2) + 4 * (L % 4) of the 32-column block n; it receives d = 32n + (lane % 32).
    const int tr_row = 4 * half + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    if (num_tiles > 0) {
        fetch(0);
        stash(0);
    }
    __syncthreads();
    for (int kt = 0; kt < num_tiles; ++kt) {
        const int buf = kt & 1;
        const int key0 = kt * kKeyTile;
        fetch(key0 + kKeyTile);  // next tile (zeros past the end), lands during this tile's math
        __builtin_amdgcn_sched_barrier(0);

        // S^T blocks s[cb][mb]: keys key0 + 32 mb + 8 (r / 4) + 4 half + r % 4 (register r) of
        // the lane's query row in column block cb.
        bf16x8 k_op[2][4];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                k_op[mb][ks] = *reinterpret_cast<const bf16x8*>(&k_tile[buf][32 * mb + col][16 * ks + 8 * half]);
        const bool need_mask = key0 + kKeyTile > safe_end;

        f32x16 s[2][2];
        bf16x8 p_op[2][4];
        auto scores = [&](int cb) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                s[cb][mb] = zero_f32x16();
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) s[cb][mb] = mfma32x32x16(k_op[mb][ks], q_op[cb][ks], s[cb][mb]);
            }
        };
        // Online softmax of one column block; P goes to bf16 operands, row sums are taken on
        // the rounded values (v_dot2 with (1, 1)) so numerator and denominator use the same P.
        auto softmax = [&](int cb) {
            if (need_mask) {
                // Register r of block mb holds key key0 + 4 half + (32 mb + 8 (r / 4) + r % 4):
                // compare the compile-time part against one per-row relative limit.
                const int limit = p.causal ? min(k_len, pos[cb] + offset + 1) : k_len;
                const int rel = limit - key0 - 4 * half;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (32 * mb + 8 * (r >> 2) + (r & 3) >= rel) s[cb][mb][r] = kNegInf;
            }
            float bmax = kNegInf;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) bmax = fmaxf(bmax, s[cb][mb][r]);
            bmax = max_xor32(bmax);
            const float tmax = bmax * c2;
            if (__any(tmax > m[cb] + kRescaleSlack)) {
                const float m_new = fmaxf(m[cb], tmax);
                const float alpha = exp2_fast(m[cb] - (m_new == kNegInf ? 0.0f : m_new));
                dsum[cb] *= alpha;
#pragma unroll
                for (int n = 0; n < 2; ++n) acc[cb][n] *= alpha;
                m[cb] = m_new;
            }
            const float neg_m = m[cb] == kNegInf ? 0.0f : -m[cb];
            float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    bf16x2 pr;
                    pr[0] = (__bf16)exp2_fast(fmaf(s[cb][mb][r], c2, neg_m));
                    pr[1] = (__bf16)exp2_fast(fmaf(s[cb][mb][r + 1], c2, neg_m));
                    // PV k-step u = 2 mb + r / 8 takes registers 8 (u % 2) .. + 7 of block mb.
                    p_op[cb][2 * mb + (r >> 3)][r & 7] = pr[0];
                    p_op[cb][2 * mb + (r >> 3)][(r & 7) + 1] = pr[1];
                    ps[r & 3 ? 1 : 0] = sum_bf16x2(pr, ps[r & 3 ? 1 : 0]);
                }
            dsum[cb] += ps[0] + ps[1];
        };
        // O^T += V^T . P^T over four 16-key steps; V^T operands by transpose reads.
        bf16x8 v_op[4][2];
        auto load_v = [&]() {
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const __bf16* vrow = &v_tile[buf][16 * u + tr_row][32 * n + tr_col];
                    const bf16x4 lo4 = lds_read_tr4(vrow);
                    const bf16x4 hi4 = lds_read_tr4(vrow + 8 * kVPitch);
                    v_op[u][n] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                }
        };
        auto pv = [&](int cb) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int n = 0; n < 2; ++n) acc[cb][n] = mfma32x32x16(v_op[u][n], p_op[cb][u], acc[cb][n]);
        };

        scores(0);
        scores(1);
        softmax(0);
        softmax(1);
        load_v();
        pv(0);
        pv(1);

        stash(buf ^ 1);  // the other buffer was released by the previous barrier
        __syncthreads();
    }

    // Epilogue: out = acc / d. Lane holds d-channels 32n + 8 (r / 4) + 4 half + r % 4.
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const float dtot = sum_xor32(dsum[cb]);
        if (!valid[cb]) continue;
        const float inv = dtot > 0.0f ? 1.0f / dtot : 0.0f;
        const int64_t obase = static_cast<int64_t>(q_start + pos[cb]) * p.o_stride_tok +
                              static_cast<int64_t>(head[cb]) * p.o_stride_head;
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int quad = 0; quad < 4; ++quad) {
                const int d0 = 32 * n + 8 * quad + 4 * half;
                if (p.out_is_bf16) {
                    bf16x4 o;
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = (__bf16)(acc[cb][n][4 * quad + i] * inv);
                    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.out) + obase + d0) = o;
                } else {
                    f32x4 o;
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = acc[cb][n][4 * quad + i] * inv;
                    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + obase + d0) = o;
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
