// Split-KV decode with a learned per-head softmax sink (gfx950).
//
// Source: "GPT-OSS on Day 0" (Perplexity), section "Kernels for GPT-OSS", subsection "Sink
// attention": attention is parallelised over heads and over the KV length; the online softmax
// keeps a running max m and running scale d per query row, m starts at the head's sink value and
// d at 1, and when the KV length is split into chunks the sink is counted in the first chunk only.
//
// Work decomposition: one work-group per (sequence b, set of one, two or four KV heads, chunk c),
// numbered with the KV-head set fastest, then the sequence, then the chunk (the (sequence, head
// set) index rotated by the chunk when the grid takes more than one round). Chunk-major order
// starts the leading chunks of every sequence (full whenever the sequence reaches past them) first,
// so with ragged lengths the short or empty trailing chunks run last and the tail is short. The
// query rows that share a KV head are the columns of the matrix-core tiles: its G = Hq/Hkv heads
// for one new token, or G x T rows when a sequence decodes T tokens at once (speculative or
// multi-token verification), column c = token c / G, head c % G, in up to four tiles of 16
// columns (columns >= G x T are padding). Every K/V byte is read from HBM once and serves all of
// them.
//
// Inside the work-group, each 64-key block of the chunk is staged in LDS once: every thread loads
// two 16-byte pieces of K rows and two of V rows (with two or four KV heads, the 256 or 512 bytes
// their slices take in a token-major cache row), and stores them into double-buffered K and V
// tiles. With more than one column tile, wave w of a KV head's team folds column tile w over every
// block of the chunk, so each wave owns the complete chunk state of its columns and no cross-wave
// reduction is needed. With one tile (G x T <= 16, e.g. one new token of 8 query heads) the four
// waves split each block's keys instead (fold_keys) and combine their states at the chunk end. The
// loads of block i + 2 are in flight while block i is folded and block i + 1 goes from registers
// into the other LDS buffer; one barrier per block. (One block ahead, or three, measured slower.)
// On a single round of paired work-groups with the key split, each wave instead loads and stages
// only its own 16 keys' rows of its own head in a private LDS region, so the loop has no barrier
// (private staging, below).
//
// With T tokens, the sequence length L counts the new tokens, and token t sees keys j <= L - T + t
// (the causal rule of the last T rows of a prefill); only the last T - 1 keys need a mask.
//
// Per block, per active wave of the column-tile fold (fold_keys does the same for 16 keys):
//   S^T (64 keys x 16 columns) = K (64 x 64) . Q^T (64 x 16): 8 MFMA 16x16x32, K operands read
//     from the K tile (lane (col, grp) reads key row 16t + col, elements 8grp and 32 + 8grp), Q^T
//     resident in registers.
//   Online softmax on S^T columns in the log2 domain (scale and sink pre-multiplied by log2 e).
//   O^T (64 d x 16 columns) += V^T (64 x 64) . P^T (64 x 16): 8 MFMA 16x16x32. P^T comes straight
//     from the S^T accumulator registers (same lanes, same columns); V^T comes from the row-major V
//     tile through the gfx950 transpose read, so no element-wise transposition is needed.

#include "chunk_merge.h"
#include "device_common.h"
#include "launch.h"
#include "plan.h"

namespace sinkattn {
namespace {

constexpr int kBlockKeys = 64;  // keys per staged block
// K tile row pitch in bf16 elements: 144 bytes, so the 16-byte reads of 16 consecutive rows start
// on 16 disjoint 4-bank groups.
constexpr int kKPitch = 72;
// V tile row pitch in bf16 elements: 64 + 16 pad = 160 bytes = 40 dwords. The transpose reads of
// 8 consecutive rows then start on 8 disjoint 8-bank groups (conflict-free per half-wave).
constexpr int kVPitch = 80;

// Online-softmax update of one 16-column tile from its S^T block (64 keys x 16 columns, lane
// (col, grp) holding keys 16t + 4grp + i): on tail blocks keys at or past `lim` are masked; the
// running max m, this lane's share of d and the O^T accumulators are updated, and P^T comes back
// as the two bf16 B operands of the PV products. P^T k-slots for key group u (32 keys): slots 0..3
// = keys 32u + 4grp + e (S^T block 2u), slots 4..7 = keys 32u + 16 + 4grp + e (S^T block 2u + 1),
// which is where this lane's S^T values already sit.
__device__ __forceinline__ void tile_softmax(const f32x4 (&s)[4], float& m, float& dsum, f32x4 (&acc)[4],
                                             bool tail, int base, int lim, float c2, int grp,
                                             bf16x8 (&p_op)[2]) {
    float x[16];
    float bmax = kNegInf;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v = s[t][i] * c2;
            if (tail && base + 16 * t + 4 * grp + i >= lim) v = kNegInf;
            x[4 * t + i] = v;
            bmax = fmaxf(bmax, v);
        }
    bmax = max_over_groups(bmax);
    const float m_new = fmaxf(m, bmax);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = exp2_fast(m - m_use);
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        x[e] = exp2_fast(x[e] - m_use);
        psum += x[e];
    }
    dsum = dsum * alpha + psum;
    m = m_new;
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[n] *= alpha;

#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p_op[u][e] = (__bf16)x[4 * (2 * u) + e];
            p_op[u][4 + e] = (__bf16)x[4 * (2 * u + 1) + e];
        }
}

// Completion of the fused kernels. Wave 0 has written every chunk state of the work-group with
// write-through stores; thread 0 (in that wave) takes a device-scope release fence (on gfx950 an L2
// write-back plus a wait for the wave's outstanding stores, so all of them are complete) and counts
// the work-group done on the counter of its (sequence, KV-head set). The last one to arrive merges
// all chunks of the set's query rows (set_rows heads x T tokens) and writes out/lse. Only the last
// arrival takes the acquire fence (an L2 and L1 invalidate), after which it reads every chunk's
// states whichever XCD produced them. Each wave merges four rows at a time (measured 0.7 us faster
// than one row per wave on 8 x 8192 keys, one token).
template <int kWaves>
__device__ __forceinline__ void fused_merge_tail(const DecodeSplitParams& p, int b, int head_set, int set_rows,
                                                 int heads_per_row, int wave_all, int& last_arrival) {
    uint32_t* counter = p.counters + static_cast<int64_t>(b) * heads_per_row + head_set;
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const bool last = atomicAdd(counter, 1u) == static_cast<uint32_t>(p.num_chunks - 1);
        if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        last_arrival = last;
    }
    __syncthreads();
    if (!last_arrival) return;
    const int lane = threadIdx.x & 63;
    const int q_len = p.q_len;
    const int rows = set_rows * q_len;
    for (int r0 = 4 * wave_all; r0 < rows; r0 += 4 * kWaves) {
        const int hl = r0 + (lane >> 4);
        if (hl >= rows) continue;
        const int tok = hl / set_rows;
        const int h = head_set * set_rows + hl % set_rows;
        const int64_t bh = (static_cast<int64_t>(b) * q_len + tok) * p.num_q_heads + h;
        f32x4 o;
        float lse;
        // hl is the same on the 16 lanes of a quarter, so whole quarters merge together.
        const float* pm = p.partial_m + bh * p.num_chunks;
        const float* pd = p.partial_d + bh * p.num_chunks;
        const float* po = p.partial_o + bh * p.num_chunks * kHeadDim;
        if (p.num_chunks <= 16)
            merge_few_chunk_states_x4(pm, pd, po, p.num_chunks, lane, o, lse);
        else
            merge_chunk_states_x4(pm, pd, po, p.num_chunks, lane, o, lse);
        const int64_t off = b * p.o_stride_b + tok * p.o_stride_tok + h * p.o_stride_head + 4 * (lane & 15);
        if (p.out_is_bf16) {
            bf16x4 ob;
#pragma unroll
            for (int e = 0; e < 4; ++e) ob[e] = (__bf16)o[e];
            *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.out) + off) = ob;
        } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + off) = o;
        }
        if (p.lse != nullptr && (lane & 15) == 0)
            p.lse[b * p.lse_stride_b + tok * p.lse_stride_tok + h * p.lse_stride_head] = lse;
    }
    // Leave the counter at zero for the next call.
    if (threadIdx.x == 0) atomicExch(counter, 0u);
}

// The 16-byte pieces of one 64-key block that a thread stages: two of K and two of V.
struct KvStage {
    bf16x8 k[2];
    bf16x8 v[2];
};

// Piece j of thread tid: index s = tid + j * 256 * kHeads over (row, head, 16-byte segment) with
// the segment fastest, then the head (adjacent 128-byte head slices), then the row. Every K/V byte
// is read once per call, so the loads carry the non-temporal hint.
template <int kHeads>
__device__ __forceinline__ void stage_load(KvStage& r, __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                           uint32_t k_row_bytes, uint32_t v_row_bytes, uint32_t base, int tid) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int piece = tid + j * kSplitThreads * kHeads;
        const uint32_t key = base + piece / (8 * kHeads);
        const uint32_t off = 16 * (piece % (8 * kHeads));
        r.k[j] = buffer_load_x8_stream(krs, key * k_row_bytes + off);
        r.v[j] = buffer_load_x8_stream(vrs, key * v_row_bytes + off);
    }
}

template <int kHeads>
__device__ __forceinline__ void stage_store(const KvStage& r, __bf16 (*kt)[kBlockKeys][kKPitch],
                                            __bf16 (*vt)[kBlockKeys][kVPitch], int tid) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int piece = tid + j * kSplitThreads * kHeads;
        const int row = piece / (8 * kHeads);
        const int hh = (piece / 8) % kHeads;
        const int seg = piece % 8;
        *reinterpret_cast<bf16x8*>(&kt[hh][row][8 * seg]) = r.k[j];
        *reinterpret_cast<bf16x8*>(&vt[hh][row][8 * seg]) = r.v[j];
    }
}

// SINKATTN_POISON_LDS builds: NaN into exactly the elements stage_store writes for this thread.
template <int kHeads>
__device__ __forceinline__ void stage_poison(__bf16 (*kt)[kBlockKeys][kKPitch], __bf16 (*vt)[kBlockKeys][kVPitch],
                                             int tid) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int piece = tid + j * kSplitThreads * kHeads;
        const int row = piece / (8 * kHeads);
        const int hh = (piece / 8) % kHeads;
        const int seg = piece % 8;
        *reinterpret_cast<bf16x8*>(&kt[hh][row][8 * seg]) = nan_bf16x8();
        *reinterpret_cast<bf16x8*>(&vt[hh][row][8 * seg]) = nan_bf16x8();
    }
}

// One wave, one column tile, one staged block: S^T from the K tile (lane (col, grp) reads key row
// 16t + col, elements 8grp and 32 + 8grp: the A operands of the 16x16x32 products), the online
// softmax, and O^T += V^T . P^T with V^T from transpose reads of the V tile: lane (grp, col) points
// at row 4grp + col/4 (+16 for slots 4..7) and columns 16n + 4(col%4), and receives column 16n + col
// of rows 4grp + 0..3.
__device__ __forceinline__ void fold_staged(float& m, float& dsum, f32x4 (&acc)[4], const __bf16 (*kt)[kKPitch],
                                            const __bf16 (*vt)[kVPitch], const bf16x8 (&q_op)[2], int base,
                                            int tail_from, int lim, float c2, int col, int grp) {
    f32x4 s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(&kt[16 * t + col][8 * grp]);
        const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(&kt[16 * t + col][32 + 8 * grp]);
        s[t] = mfma16x16x32(k0, q_op[0], zero_f32x4());
        s[t] = mfma16x16x32(k1, q_op[1], s[t]);
    }
    bf16x8 p_op[2];
    tile_softmax(s, m, dsum, acc, base + kBlockKeys > tail_from, base, lim, c2, grp, p_op);
    const int tr_row = 4 * grp + (col >> 2);
    const int tr_col = 4 * (col & 3);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const bf16x4 lo4 = lds_read_tr4(&vt[32 * u + tr_row][16 * n + tr_col]);
            const bf16x4 hi4 = lds_read_tr4(&vt[32 * u + 16 + tr_row][16 * n + tr_col]);
            const bf16x8 v_op = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            acc[n] = mfma16x16x32(v_op, p_op[u], acc[n]);
        }
}

// Key-split fold, for one column tile (G x T <= 16): wave w of a KV head's team takes keys
// [16w, 16w + 16) of every staged block, so all four waves share each block's work and each keeps
// its own state (m, d, O^T) over its keys. S^T (16 keys x 16 columns) = 2 MFMA 16x16x32 with K
// operands from rows 16w + col of the K tile; the lane's 4 scores (keys 16w + 4grp + i) are, once
// exponentiated, the B operand of v_mfma_f32_16x16x16_bf16, and V^T (64 d x 16 keys) comes from
// transpose reads of the V tile: O^T += V^T . P^T in 4 MFMA 16x16x16.
// The operands of one wave's key-split fold of a block: its two K A-operands (key rows 16w + col,
// elements 8grp and 32 + 8grp) and the four V^T A-operands of the 16x16x16 products (transpose
// reads: lane (grp, col) points at row 16w + 4grp + col/4, columns 16n + 4(col%4)).
struct KeyOps {
    bf16x8 k[2];
    bf16x4 v[4];
};

__device__ __forceinline__ void fold_key_ops(float& m, float& dsum, f32x4 (&acc)[4], const KeyOps& ops,
                                             const bf16x8 (&q_op)[2], int base, int tail_from, int lim, float c2,
                                             int grp, int w) {
    f32x4 s = mfma16x16x32(ops.k[0], q_op[0], zero_f32x4());
    s = mfma16x16x32(ops.k[1], q_op[1], s);
    const bool tail = base + kBlockKeys > tail_from;
    float x[4];
    float bmax = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float v = s[i] * c2;
        if (tail && base + 16 * w + 4 * grp + i >= lim) v = kNegInf;
        x[i] = v;
        bmax = fmaxf(bmax, v);
    }
    bmax = max_over_groups(bmax);
    const float m_new = fmaxf(m, bmax);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = exp2_fast(m - m_use);
    bf16x4 p_op;
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = exp2_fast(x[i] - m_use);
        psum += x[i];
        p_op[i] = (__bf16)x[i];
    }
    dsum = dsum * alpha + psum;
    m = m_new;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        acc[n] *= alpha;
        acc[n] = mfma16x16x16(ops.v[n], p_op, acc[n]);
    }
}

__device__ __forceinline__ void fold_keys(float& m, float& dsum, f32x4 (&acc)[4], const __bf16 (*kt)[kKPitch],
                                          const __bf16 (*vt)[kVPitch], const bf16x8 (&q_op)[2], int base,
                                          int tail_from, int lim, float c2, int col, int grp, int w) {
    KeyOps ops;
    ops.k[0] = *reinterpret_cast<const bf16x8*>(&kt[16 * w + col][8 * grp]);
    ops.k[1] = *reinterpret_cast<const bf16x8*>(&kt[16 * w + col][32 + 8 * grp]);
    const int tr_row = 16 * w + 4 * grp + (col >> 2);
    const int tr_col = 4 * (col & 3);
#pragma unroll
    for (int n = 0; n < 4; ++n) ops.v[n] = lds_read_tr4(&vt[tr_row][16 * n + tr_col]);
    fold_key_ops(m, dsum, acc, ops, q_op, base, tail_from, lim, c2, grp, w);
}

template <int kHeads, bool kFused, bool kKeySplit, bool kPrivate>
__global__ __launch_bounds__(kSplitThreads * kHeads) void decode_split_bf16_kernel(DecodeSplitParams p) {
    static_assert(kKeySplit || !kPrivate, "private staging serves the key split");
    constexpr int kWaves = kSplitWaves * kHeads;
    __shared__ int last_arrival;
    __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][kHeads][kBlockKeys][kKPitch];
    __shared__ __attribute__((aligned(16))) __bf16 v_lds[2][kHeads][kBlockKeys][kVPitch];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hsub = wave_all / kSplitWaves;  // which of the work-group's KV heads
    const int tile = wave_all % kSplitWaves;  // this wave's column tile
    const int col = lane & 15;
    const int grp = lane >> 4;

    // Chunk-major: chunk = blockIdx / R with R = batch x head sets. When the grid takes more than
    // one round of work-groups, the (sequence, head set) index r within a chunk is rotated by the
    // chunk, r = (blockIdx - chunk) mod R: work-groups go to the eight XCDs round-robin by
    // blockIdx, so without the rotation every chunk of a sequence lands on the same XCD and an
    // XCD's share of the keys is the sum of its sequences' lengths (128 sequences of 1-8192 keys:
    // XCDs finished 16% apart, 199 us; rotated 189 us); with it chunk c of row r runs on XCD
    // (r + c) mod 8 when R is a multiple of 8. A single round keeps the plain order, in which the
    // work-groups running together read adjacent pieces of the same cache rows (8 x 8192 keys:
    // 25.2 us plain, 26.4 us rotated, 27.0 us with the sequence fastest).
    const int heads_per_row = p.num_kv_heads / kHeads;
    const int rows_per_chunk = p.batch * heads_per_row;
    const int chunk = static_cast<int>(blockIdx.x) / rows_per_chunk;
    const int rotate = static_cast<int64_t>(gridDim.x) > kComputeUnits ? chunk % rows_per_chunk : 0;
    int bid = static_cast<int>(blockIdx.x) % rows_per_chunk - rotate;
    bid += bid < 0 ? rows_per_chunk : 0;
    const int head_set = bid % heads_per_row;
    const int g = head_set * kHeads + hsub;
    const int b = bid / heads_per_row;
    const int group = p.num_q_heads / p.num_kv_heads;
    const int q_len = p.q_len;
    const int columns = group * q_len;

    int len = p.seqlens_k[b];
    len = len < 0 ? 0 : (len > p.capacity ? static_cast<int>(p.capacity) : len);
    const int64_t lo = static_cast<int64_t>(chunk) * p.chunk_size;
    const int64_t hi = lo + p.chunk_size < len ? lo + p.chunk_size : len;
    const int first_lim = len - q_len + 1;
    const int tail_from = first_lim < hi ? first_lim : static_cast<int>(hi);

    // This wave's 16 columns: column c = token c / G, head c % G of KV head g. With the key split
    // every wave of the team works on the one tile (and wave 0 writes the combined state).
    const bool active = kKeySplit || 16 * tile < columns;
    const bool writes_state = kKeySplit ? tile == 0 : active;
    const int c = (kKeySplit ? 0 : 16 * tile) + col;
    const bool col_valid = c < columns;
    const int tok = col_valid ? c / group : 0;
    const int head = g * group + (col_valid ? c % group : 0);
    const __bf16* qrow = static_cast<const __bf16*>(p.q) + b * p.q_stride_b + tok * p.q_stride_tok +
                         head * p.q_stride_head;
    bf16x8 q_op[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        q_op[h] = col_valid ? *reinterpret_cast<const bf16x8*>(qrow + 32 * h + 8 * grp) : zero_bf16x8();
    const int tok_lim = first_lim + tok;
    const int lim = tok_lim < hi ? tok_lim : static_cast<int>(hi);
    const float c2 = p.scale * kLog2e;
    // Every wave covers the whole chunk for its columns, so each starts chunk 0 from the sink; with
    // the key split the waves hold parts of one state, and only wave 0 carries the sink.
    float m = kNegInf, dsum = 0.0f;
    if ((chunk == 0 || kMutateSinkEveryChunk) && (!kKeySplit || tile == 0)) {
        m = p.sinks[head] * kLog2e;
        dsum = (grp == 0 && m != kNegInf && !kMutateD0Zero) ? 1.0f : 0.0f;
    }
    f32x4 acc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[n] = zero_f32x4();

    // Buffer ranges end at the chunk end (rows [0, hi) of the work-group's KV-head slices; with two
    // heads their slices are adjacent in each row).
    const int g0 = head_set * kHeads;
    const __bf16* kbase = static_cast<const __bf16*>(p.k) + b * p.k_stride_b + g0 * p.k_stride_head;
    const __bf16* vbase = static_cast<const __bf16*>(p.v) + b * p.v_stride_b + g0 * p.v_stride_head;
    const uint32_t k_row_bytes = static_cast<uint32_t>(p.k_stride_tok * 2);
    const uint32_t v_row_bytes = static_cast<uint32_t>(p.v_stride_tok * 2);
    const __amdgpu_buffer_rsrc_t krs = make_buffer(kbase, static_cast<uint32_t>(hi) * k_row_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_buffer(vbase, static_cast<uint32_t>(hi) * v_row_bytes);

    const int blocks = hi > lo ? static_cast<int>((hi - lo + kBlockKeys - 1) / kBlockKeys) : 0;
    const uint32_t base0 = static_cast<uint32_t>(lo);
    if constexpr (kPoisonLds) {
        bf16x8* kz = reinterpret_cast<bf16x8*>(&k_lds[0][0][0][0]);
        bf16x8* vz = reinterpret_cast<bf16x8*>(&v_lds[0][0][0][0]);
        for (int i = tid; i < static_cast<int>(sizeof(k_lds) / 16); i += kSplitThreads * kHeads) kz[i] = nan_bf16x8();
        for (int i = tid; i < static_cast<int>(sizeof(v_lds) / 16); i += kSplitThreads * kHeads) vz[i] = nan_bf16x8();
        __syncthreads();
    }
    if constexpr (kPrivate) {
        // Private staging (key split, one round of work-groups): wave w of a KV head's team folds
        // keys [16w, 16w + 16) of every block, so it loads, stages and reads only those 16 rows of
        // its own head (2 KB of K and 2 KB of V per block, in a region of LDS no other wave touches)
        // and no barrier is needed in the loop: a wave's LDS accesses execute in order, so the
        // store of block i + 1 lands after the fold's reads of block i. Rows are 128 bytes, 16-byte
        // chunk c of row r at position c ^ ((r >> 1) & 7) for K (the 16 rows' operand reads hit 16
        // different bank groups) and c ^ (((r >> 1) & 3) << 1) for V (the transpose reads of 8 rows
        // by two chunks likewise). Measured on 8 x 8192 keys against the shared staging below:
        // split + merge 25.9 vs 26.9 us; on the multi-round grids of four heads it was 7-8% slower
        // (the shared staging reads 512 contiguous bytes of each row per instruction), so those keep
        // the shared form.
        __bf16* pk = reinterpret_cast<__bf16*>(&k_lds[0][0][0][0]) + wave_all * (2 * 16 * kHeadDim);
        __bf16* pv = pk + 16 * kHeadDim;
        static_assert(sizeof(k_lds) >= sizeof(__bf16) * kWaves * 2 * 16 * kHeadDim, "private regions");
        uint32_t k_off[2], v_off[2];
        int st_k[2], st_v[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int piece = lane + 64 * j;
            const int r = piece >> 3, ch = piece & 7;
            k_off[j] = static_cast<uint32_t>(16 * tile + r) * k_row_bytes + 128u * hsub + 16u * ch;
            v_off[j] = static_cast<uint32_t>(16 * tile + r) * v_row_bytes + 128u * hsub + 16u * ch;
            st_k[j] = r * kHeadDim + 8 * (ch ^ ((r >> 1) & 7));
            st_v[j] = r * kHeadDim + 8 * (ch ^ (((r >> 1) & 3) << 1));
        }
        auto pload = [&](KvStage& st, int blk) {
            const uint32_t key = base0 + static_cast<uint32_t>(kBlockKeys * blk);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                st.k[j] = buffer_load_x8_stream(krs, key * k_row_bytes + k_off[j]);
                st.v[j] = buffer_load_x8_stream(vrs, key * v_row_bytes + v_off[j]);
            }
        };
        auto pstore = [&](const KvStage& st) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                *reinterpret_cast<bf16x8*>(pk + st_k[j]) = st.k[j];
                *reinterpret_cast<bf16x8*>(pv + st_v[j]) = st.v[j];
            }
        };
        const int v_row = 4 * grp + (col >> 2);
        const int v_at = v_row * kHeadDim + 4 * (col & 1);
        const int v_swz = ((v_row >> 1) & 3) << 1;
        const int v_chunk = (col & 3) >> 1;
        auto pfold = [&](int i) {
            KeyOps ops;
            ops.k[0] = *reinterpret_cast<const bf16x8*>(pk + col * kHeadDim + 8 * (grp ^ ((col >> 1) & 7)));
            ops.k[1] = *reinterpret_cast<const bf16x8*>(pk + col * kHeadDim + 8 * ((4 + grp) ^ ((col >> 1) & 7)));
#pragma unroll
            for (int n = 0; n < 4; ++n) ops.v[n] = lds_read_tr4(pv + v_at + 8 * ((2 * n + v_chunk) ^ v_swz));
            fold_key_ops(m, dsum, acc, ops, q_op, static_cast<int>(base0) + kBlockKeys * i, tail_from, lim, c2, grp,
                         tile);
        };
        // One block in flight during each fold (the loads of block i + 1, issued before it): with two
        // the split took 24.4-24.7 us instead of 23.4-23.6 on 8 x 8192 keys, as a plain read of the
        // same pattern is faster with 32 KB than with 64 KB in flight per compute unit. The
        // scheduling barriers keep the loads ahead of the fold (with no s_barrier in the loop the
        // compiler would otherwise move them).
        KvStage ra;
        pload(ra, 0);
        pstore(ra);
        for (int i = 0; i < blocks; ++i) {
            pload(ra, i + 1);
            __builtin_amdgcn_sched_barrier(0);
            pfold(i);
            pstore(ra);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Every wave is done with its private region before the tiles are reused below.
        __syncthreads();
    } else {
        KvStage ra, rb;
        stage_load<kHeads>(ra, krs, vrs, k_row_bytes, v_row_bytes, base0, tid);
        stage_store<kHeads>(ra, k_lds[0], v_lds[0], tid);
        stage_load<kHeads>(ra, krs, vrs, k_row_bytes, v_row_bytes, base0 + kBlockKeys, tid);
        __syncthreads();
        // Blocks past the chunk end load as zeros without touching memory; the loop stops before
        // folding them.
        for (int i = 0; i < blocks;) {
            if constexpr (kPoisonLds) stage_poison<kHeads>(k_lds[(i + 1) & 1], v_lds[(i + 1) & 1], tid);
            stage_load<kHeads>(rb, krs, vrs, k_row_bytes, v_row_bytes, base0 + kBlockKeys * (i + 2), tid);
            if constexpr (kKeySplit)
                fold_keys(m, dsum, acc, k_lds[i & 1][hsub], v_lds[i & 1][hsub], q_op,
                          static_cast<int>(base0) + kBlockKeys * i, tail_from, lim, c2, col, grp, tile);
            else if (active)
                fold_staged(m, dsum, acc, k_lds[i & 1][hsub], v_lds[i & 1][hsub], q_op,
                            static_cast<int>(base0) + kBlockKeys * i, tail_from, lim, c2, col, grp);
            stage_store<kHeads>(ra, k_lds[(i + 1) & 1], v_lds[(i + 1) & 1], tid);
            __syncthreads();
            if (++i >= blocks) break;
            if constexpr (kPoisonLds) stage_poison<kHeads>(k_lds[(i + 1) & 1], v_lds[(i + 1) & 1], tid);
            stage_load<kHeads>(ra, krs, vrs, k_row_bytes, v_row_bytes, base0 + kBlockKeys * (i + 2), tid);
            if constexpr (kKeySplit)
                fold_keys(m, dsum, acc, k_lds[i & 1][hsub], v_lds[i & 1][hsub], q_op,
                          static_cast<int>(base0) + kBlockKeys * i, tail_from, lim, c2, col, grp, tile);
            else if (active)
                fold_staged(m, dsum, acc, k_lds[i & 1][hsub], v_lds[i & 1][hsub], q_op,
                            static_cast<int>(base0) + kBlockKeys * i, tail_from, lim, c2, col, grp);
            stage_store<kHeads>(rb, k_lds[(i + 1) & 1], v_lds[(i + 1) & 1], tid);
            __syncthreads();
            ++i;
        }
    
}
    if constexpr (kKeySplit) {
        // Combine the team's four states in the (now free) V tiles, a quarter of O^T per wave:
        // every wave publishes m and d of its 16 columns and its four 16-row blocks of O^T; wave w
        // then rescales block w of all four states to the common maximum and sums them, so it
        // holds rows [16w, 16w + 16) of each column's combined O^T in acc[0], and every wave the
        // combined d (on group 0, as the fold keeps it) and m.
        constexpr int kStateFloats = 4 * 16 * 2 + 4 * 4 * 64 * 4;
        static_assert(sizeof(v_lds) >= sizeof(float) * kHeads * kStateFloats, "state space");
        float* st = reinterpret_cast<float*>(&v_lds[0][0][0][0]) + hsub * kStateFloats;
        f32x4* parts = reinterpret_cast<f32x4*>(st + 4 * 16 * 2);
        const float d_wave = sum_over_groups(dsum);
        if (grp == 0) *reinterpret_cast<f32x2*>(&st[2 * (16 * tile + col)]) = f32x2{m, d_wave};
#pragma unroll
        for (int n = 0; n < 4; ++n) parts[(4 * n + tile) * 64 + lane] = acc[n];
        __syncthreads();
        float mw[4], dw[4];
        float big = kNegInf;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const f32x2 md = *reinterpret_cast<const f32x2*>(&st[2 * (16 * w + col)]);
            mw[w] = md[0];
            dw[w] = md[1];
            big = fmaxf(big, mw[w]);
        }
        float d_all = 0.0f;
        f32x4 o = zero_f32x4();
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float sc = mw[w] == kNegInf ? 0.0f : exp2_fast(mw[w] - big);
            d_all += dw[w] * sc;
            o += sc * parts[(4 * tile + w) * 64 + lane];
        }
        acc[0] = o;
        m = big;
        dsum = grp == 0 ? d_all : 0.0f;
    }

    // The chunk state of each valid column: o = acc / d, m (natural log), d.
    const float d_tot = sum_over_groups(dsum);
    const float inv = d_tot > 0.0f ? 1.0f / d_tot : 0.0f;
    const float m_nat = d_tot > 0.0f ? m * kLn2 : kNegInf;
    const int64_t row = ((static_cast<int64_t>(b) * q_len + tok) * p.num_q_heads + head) * p.num_chunks + chunk;
    if constexpr (kFused) {
        // Every chunk state of the work-group goes through LDS (the K tiles are free after the
        // loop's last barrier) and wave 0 alone writes them all with write-through stores, one
        // contiguous 256-byte row of partial_o per store instruction; the release fence of that
        // same wave in fused_merge_tail then orders all of them before the arrival count.
        constexpr int kOPitch = kHeadDim + 4;
        static_assert(sizeof(k_lds) >= sizeof(float) * kWaves * 16 * (kOPitch + 2), "staging space");
        float (*ot_all)[kOPitch] = reinterpret_cast<float (*)[kOPitch]>(&k_lds[0][0][0][0]);
        float* md_all = reinterpret_cast<float*>(&k_lds[0][0][0][0]) + kWaves * 16 * kOPitch;
        if (kKeySplit || writes_state) {
            float (*ot)[kOPitch] = ot_all + 16 * (kKeySplit ? hsub * kSplitWaves : wave_all);
            if constexpr (kKeySplit)
                *reinterpret_cast<f32x4*>(&ot[col][16 * tile + 4 * grp]) = acc[0] * inv;
            else
#pragma unroll
                for (int n = 0; n < 4; ++n) *reinterpret_cast<f32x4*>(&ot[col][16 * n + 4 * grp]) = acc[n] * inv;
            if (writes_state && grp == 0) {
                md_all[(2 * wave_all) * 16 + col] = m_nat;
                md_all[(2 * wave_all + 1) * 16 + col] = d_tot;
            }
        }
        __syncthreads();
        if (wave_all == 0) {
            for (int w = 0; w < kWaves; ++w) {
                const int w_tile = w % kSplitWaves;
                const bool w_writes = kKeySplit ? w_tile == 0 : 16 * w_tile < columns;
                if (!w_writes) continue;
                const int w_g = head_set * kHeads + w / kSplitWaves;
                const int c0 = kKeySplit ? 0 : 16 * w_tile;
                const int tile_cols = columns - c0 < 16 ? columns - c0 : 16;
                auto state_row = [&](int r) {
                    const int cr = c0 + r;
                    return ((static_cast<int64_t>(b) * q_len + cr / group) * p.num_q_heads + w_g * group + cr % group) *
                               p.num_chunks + chunk;
                };
                // Two rows per store instruction (8 bytes a lane); all LDS reads of the tile are
                // issued before its stores, so the wave waits for LDS once per tile.
                uint64_t two[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = 2 * i + (lane >> 5);
                    two[i] = r < tile_cols ? *reinterpret_cast<const uint64_t*>(&ot_all[16 * w + r][2 * (lane & 31)]) : 0;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = 2 * i + (lane >> 5);
                    if (r < tile_cols)
                        __hip_atomic_store(reinterpret_cast<uint64_t*>(&p.partial_o[state_row(r) * kHeadDim + 2 * (lane & 31)]),
                                           two[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                }
                if (lane < tile_cols) {
                    const int64_t row_l = state_row(lane);
                    __hip_atomic_store(&p.partial_m[row_l], md_all[(2 * w) * 16 + lane], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_SYSTEM);
                    __hip_atomic_store(&p.partial_d[row_l], md_all[(2 * w + 1) * 16 + lane], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_SYSTEM);
                }
            }
        }
    } else if (kKeySplit && col_valid) {
        *reinterpret_cast<f32x4*>(p.partial_o + row * kHeadDim + 16 * tile + 4 * grp) = acc[0] * inv;
        if (tile == 0 && grp == 0) {
            p.partial_m[row] = m_nat;
            p.partial_d[row] = d_tot;
        }
    } else if (writes_state && col_valid) {
        float* orow = p.partial_o + row * kHeadDim + 4 * grp;
#pragma unroll
        for (int n = 0; n < 4; ++n) *reinterpret_cast<f32x4*>(orow + 16 * n) = acc[n] * inv;
        if (grp == 0) {
            p.partial_m[row] = m_nat;
            p.partial_d[row] = d_tot;
        }
    }
    if constexpr (kFused)
        fused_merge_tail<kWaves>(p, b, head_set, kHeads * group, heads_per_row, wave_all, last_arrival);
}

// fp32 reference variant: one thread per (b, token, query head, chunk), keys visited one at a time
// with the page's online recurrence (tile of one key). Written for clarity, not speed.
__global__ __launch_bounds__(256) void decode_split_f32_kernel(DecodeSplitParams p) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = static_cast<int64_t>(p.batch) * p.q_len * p.num_q_heads * p.num_chunks;
    if (idx >= total) return;
    const int chunk = static_cast<int>(idx % p.num_chunks);
    const int head = static_cast<int>((idx / p.num_chunks) % p.num_q_heads);
    const int64_t bt = idx / (static_cast<int64_t>(p.num_chunks) * p.num_q_heads);
    const int tok = static_cast<int>(bt % p.q_len);
    const int b = static_cast<int>(bt / p.q_len);
    const int g = head / (p.num_q_heads / p.num_kv_heads);

    int len = p.seqlens_k[b];
    len = len < 0 ? 0 : (len > p.capacity ? static_cast<int>(p.capacity) : len);
    const int64_t lo = static_cast<int64_t>(chunk) * p.chunk_size;
    // Token tok sees keys below len - q_len + 1 + tok.
    const int64_t tok_end = static_cast<int64_t>(len) - p.q_len + 1 + tok;
    int64_t hi = lo + p.chunk_size < len ? lo + p.chunk_size : len;
    hi = hi < tok_end ? hi : tok_end;

    const float* qrow = static_cast<const float*>(p.q) + b * p.q_stride_b + tok * p.q_stride_tok +
                        head * p.q_stride_head;
    float qv[kHeadDim], acc[kHeadDim];
    for (int d = 0; d < kHeadDim; ++d) {
        qv[d] = qrow[d];
        acc[d] = 0.0f;
    }
    float m = kNegInf, dsum = 0.0f;
    if (chunk == 0 || kMutateSinkEveryChunk) {
        m = p.sinks[head];
        dsum = (m == kNegInf || kMutateD0Zero) ? 0.0f : 1.0f;
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
    const int64_t row = idx;  // ((b, token), head, chunk) row-major == idx
    const float inv = dsum > 0.0f ? 1.0f / dsum : 0.0f;
    for (int d = 0; d < kHeadDim; ++d) p.partial_o[row * kHeadDim + d] = acc[d] * inv;
    p.partial_m[row] = dsum > 0.0f ? m : kNegInf;
    p.partial_d[row] = dsum;
}

}  // namespace

// Launches the kernel instance decode_shape (plan.h) names: KV heads per work-group, key split,
// single launch or not.
template <int kHeads, bool kFused>
hipError_t launch_split_heads(const DecodeSplitParams& p, const DecodeShape& s, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(s.groups)), block(static_cast<unsigned>(s.block));
    if (s.private_staging) {
        if constexpr (kHeads == 2) decode_split_bf16_kernel<2, kFused, true, true><<<grid, block, 0, stream>>>(p);
        else return hipErrorInvalidValue;  // the plan never asks for it
    } else if (s.key_split) {
        decode_split_bf16_kernel<kHeads, kFused, true, false><<<grid, block, 0, stream>>>(p);
    } else {
        decode_split_bf16_kernel<kHeads, kFused, false, false><<<grid, block, 0, stream>>>(p);
    }
    return hipGetLastError();
}

template <bool kFused>
hipError_t launch_split(const DecodeSplitParams& p, hipStream_t stream) {
    const DecodeShape s = decode_shape(p);
    if (s.heads == 4) return launch_split_heads<4, kFused>(p, s, stream);
    if (s.heads == 2) return launch_split_heads<2, kFused>(p, s, stream);
    return launch_split_heads<1, kFused>(p, s, stream);
}

hipError_t launch_decode_split_bf16(const DecodeSplitParams& p, hipStream_t stream) {
    return launch_split<false>(p, stream);
}

hipError_t launch_decode_fused_bf16(const DecodeSplitParams& p, hipStream_t stream) {
    return launch_split<true>(p, stream);
}

hipError_t launch_decode_split_f32(const DecodeSplitParams& p, hipStream_t stream) {
    const Launch l = plan_decode_split_f32(p);
    decode_split_f32_kernel<<<dim3(static_cast<unsigned>(l.grid)), dim3(l.block), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace sinkattn
