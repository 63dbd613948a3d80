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
//   online softmax per row in the log2 domain (scale and sink multiplied by log2 e in fp32).
//     Causal mask only on the tiles that cross the diagonal or the sequence end, which come
//     last and run in a loop of their own.
//   On tiles where the softmax needs no row max (zero reference, below), the MFMA chains and
//   the exponentials are interleaved by hand so that the wave keeps its matrix and vector
//   pipes busy together.
//   O^T (64 d x 64 rows) += V^T . P^T: 16 MFMA. The S^T accumulator lanes are exactly the P^T
//     operand lanes, so P never leaves registers; V stays row-major in LDS and comes back
//     transposed through ds_read_b64_tr_b16.
// K/V tiles go from memory straight into three LDS buffers (buffer_load ... lds), two tiles
// ahead of the one being multiplied, one barrier per tile. The bf16 output leaves through LDS as
// whole 128-byte rows.
// Work-groups are numbered query-tile-major with the KV head fastest, so consecutive
// work-groups (which the dispatcher spreads over the eight XCDs) read different KV heads and each
// XCD's L2 keeps re-serving one head's K/V. Within a sequence, tiles are issued last-position
// first: the longest causal rows start earliest.

#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "plan.h"

namespace sinkattn {
namespace {

// The kernel's lambdas are inlined by force: an outlined tile body becomes a call with its
// registers spilled to the stack.
#define SA_INLINE __attribute__((always_inline))

constexpr int kKeyTile = 64;
// K and V tiles sit in LDS unpadded (64 keys x 128-byte rows) in three buffers, written straight
// from global memory by buffer_load ... lds (no staging registers), one tile two tiles ahead of
// the one being computed. Within a row, 16-byte chunk c of K sits at chunk position
// c ^ ((row >> 1) & 7), so the 16-byte operand reads of 16 consecutive rows hit distinct banks;
// chunk c of V sits at c ^ (((row >> 1) & 1) << 2), so each transpose read (four consecutive rows,
// four chunks) hits distinct banks.
constexpr int kTileElems = kKeyTile * 64;
constexpr int kStages = 3;
// Softmax reference. Each row keeps a reference m; p = exp2(s - m) and d, O are kept relative
// to it, so any m that keeps p away from fp32/bf16 overflow and underflow gives the same
// out = O / d (the common factor 2^-m cancels). Two regimes:
//  * running-max tiles: m is the running max, raised (and O, d rescaled) only when a tile's max
//    exceeds it by more than kRescaleSlack log2 units, so p <= 2^8;
//  * zero-reference tiles: once the running max of a row lies in [-kZeroRefLimit, kZeroRefLimit]
//    (from the start, when the sink does) the row is rescaled once to m = 0, and while every row
//    of a wave has m = 0 its tiles need
//    neither a row max nor a subtraction: p = exp2(s). The row's largest contribution so far is
//    then at least 2^-kZeroRefLimit, so nothing that matters can underflow; overflow is checked
//    once at the end: a work-group in which any row's d exceeds kFastSumLimit (every p is at
//    most d) or any d or O is not finite is recomputed with running-max tiles only.
constexpr float kRescaleSlack = 8.0f;
constexpr float kZeroRefLimit = 16.0f;
constexpr float kFastSumLimit = 18446744073709551616.0f;  // 2^64

// Maps a linear query-tile index to its sequence and first position. Sequence s owns tile indices
// [V(s), V(s + 1)) with V(s) = floor(start(s) / P) + s (P positions per tile): V(s + 1) - V(s) =
// floor(end / P) - floor(start / P) + 1 >= ceil(len / P), so each sequence has room for its tiles
// plus at most one padding index, V(B) <= ceil(Tq / P) + B bounds the grid, and V(s) needs only
// start(s), so the search is parallel: each step the 64 lanes test 64 evenly spaced sequences with
// one load each and keep the last one whose V is at most the tile index (V grows with s). Within a
// sequence index 0 is the tile holding the last positions. The lanes of the last step also read
// the sequence's key bounds, so every prefix sum the work-group needs arrives in one round trip.
// Returns false for padding indices. Starts and lengths are clamped to [0, total) so that broken
// prefix sums cannot move a row out of bounds (the tiles then computed are unspecified).
struct TileSpan {
    int seq, first_pos, q_start, q_len, k_start, k_len;
};

__device__ bool locate_tile(const int32_t* cu_q, const int32_t* cu_k, int num_seqs, int total_q, int total_k,
                            int positions_per_tile, int tile, int lane, TileSpan& t) {
    auto clamp_start = [](int x, int total) { return min(max(x, 0), total); };
    int lo = 0, n = num_seqs;
    // This lane's probe of the last step: prefix sums at s and s + 1 (raw, clamped below).
    int q0 = 0, q1 = 0, k0 = 0, k1 = 0;
    int last = 0;  // lane whose probe is the sequence found
    bool probed = false;
    while (n > 1) {
        const int step = (n + 63) >> 6;
        const int s = lo + lane * step;
        bool ok = false;
        if (s < lo + n) {
            q0 = cu_q[s];
            q1 = cu_q[s + 1];
            k0 = cu_k[s];
            k1 = cu_k[s + 1];
            ok = clamp_start(q0, total_q) / positions_per_tile + s <= tile;
        }
        // Lane 0 tests lo, whose V is at most the tile index for well-formed prefix sums.
        const int k = max(__popcll(__ballot(ok)), 1);
        lo += (k - 1) * step;
        n = min(step, n - (k - 1) * step);
        last = k - 1;
        probed = true;
    }
    int sq0, sq1, sk0, sk1;
    if (probed) {
        sq0 = __builtin_amdgcn_readlane(q0, last);
        sq1 = __builtin_amdgcn_readlane(q1, last);
        sk0 = __builtin_amdgcn_readlane(k0, last);
        sk1 = __builtin_amdgcn_readlane(k1, last);
    } else {
        sq0 = cu_q[0];
        sq1 = cu_q[1];
        sk0 = cu_k[0];
        sk1 = cu_k[1];
    }
    t.seq = lo;
    t.q_start = clamp_start(sq0, total_q);
    t.q_len = min(max(sq1 - t.q_start, 0), total_q - t.q_start);
    t.k_start = clamp_start(sk0, total_k);
    t.k_len = min(max(sk1 - t.k_start, 0), total_k - t.k_start);
    const int tiles = (t.q_len + positions_per_tile - 1) / positions_per_tile;
    const int local = tile - (t.q_start / positions_per_tile + lo);
    if (local < 0 || local >= tiles) return false;
    t.first_pos = (tiles - 1 - local) * positions_per_tile;
    return true;
}

template <bool kSplit>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_bf16_kernel(PrefillParams p) {
    __shared__ __attribute__((aligned(16))) __bf16 k_lds[kStages][kTileElems];
    __shared__ __attribute__((aligned(16))) __bf16 v_lds[kStages][kTileElems];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;   // MFMA column: query row within a 32-row block
    const int half = lane >> 5;  // k-slot group

    // Work-group order: KV head fastest, then (split-KV prefill) the split, then the query tile.
    int bid = blockIdx.x;
    const int g = bid % p.num_kv_heads;
    bid /= p.num_kv_heads;
    int split = 0;
    if constexpr (kSplit) {
        split = bid % p.num_splits;
        bid /= p.num_splits;
    }
    const int tile = bid;
    const int group = p.num_q_heads / p.num_kv_heads;
    const int positions_per_tile = kRowsPerTile / group;

    TileSpan span;
    if (!locate_tile(p.cu_seqlens_q, p.cu_seqlens_k, p.num_seqs, static_cast<int>(p.total_q),
                     static_cast<int>(p.total_k), positions_per_tile, tile, lane, span))
        return;
    const int first_pos = span.first_pos, q_start = span.q_start, q_len = span.q_len;
    const int k_start = span.k_start, k_len = span.k_len;
    const int offset = k_len - q_len;  // bottom-right causal alignment

    // Rows of this lane: column block cb -> tile row 64 wave + 32 cb + col. S^T comes out of the
    // MFMA exact (fp32 sums of bf16 products); scale * log2 e is applied in fp32 per score.
    int pos[2], head[2];
    bool valid[2];
    const float c2 = p.scale * kLog2e;
    bf16x8 q_op[2][4];
    float sink2[2];
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
        sink2[cb] = p.sinks[head[cb]] * kLog2e;
    }

    // Keys this tile's rows may see: [0, key_end).
    const int last_pos = min(first_pos + positions_per_tile, q_len) - 1;
    int key_end = p.causal ? min(k_len, last_pos + offset + 1) : k_len;
    key_end = key_end < 0 ? 0 : key_end;
    // Keys below safe_end are visible to every row of the tile: KV tiles [0, mask_from) need no
    // mask (the diagonal and the sequence end fall in the tiles after them).
    const int safe_end = p.causal ? min(k_len, first_pos + offset + 1) : k_len;
    const int num_tiles = (key_end + kKeyTile - 1) / kKeyTile;
    const int mask_from = min(num_tiles, max(safe_end, 0) / kKeyTile);
    // KV tiles of this work-group: all of them, or (split-KV prefill) those of its split, whose
    // boundaries fall on whole tiles except at the sequence end. Only split 0 carries the sink.
    int kt_begin = 0, kt_end = num_tiles;
    bool carries_sink = true;
    if constexpr (kSplit) {
        const int per = (k_len + p.num_splits - 1) / p.num_splits;
        const int split_keys = (per + kKeyTile - 1) / kKeyTile * kKeyTile;
        const int lo = min(split * split_keys, k_len);
        const int hi = min(lo + split_keys, k_len);
        // A non-empty split starts at split * split_keys < Lk, a whole tile; an empty one (lo
        // clamped to Lk, which may fall inside a tile) processes no tile at all.
        kt_begin = lo / kKeyTile;
        kt_end = hi > lo ? max(kt_begin, min(num_tiles, (hi + kKeyTile - 1) / kKeyTile)) : kt_begin;
        carries_sink = split == 0 || kMutateSinkEveryChunk;
    }

    // K/V rows [0, key_end) of KV head g of this sequence; loads past the end return zeros.
    const __bf16* kbase = static_cast<const __bf16*>(p.k) + static_cast<int64_t>(k_start) * p.k_stride_tok +
                          static_cast<int64_t>(g) * p.k_stride_head;
    const __bf16* vbase = static_cast<const __bf16*>(p.v) + static_cast<int64_t>(k_start) * p.v_stride_tok +
                          static_cast<int64_t>(g) * p.v_stride_head;
    const uint32_t k_row_bytes = static_cast<uint32_t>(p.k_stride_tok * 2);
    const uint32_t v_row_bytes = static_cast<uint32_t>(p.v_stride_tok * 2);
    const __amdgpu_buffer_rsrc_t krs = make_buffer(kbase, static_cast<uint32_t>(key_end) * k_row_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_buffer(vbase, static_cast<uint32_t>(key_end) * v_row_bytes);

    // Staging: per tile, wave w loads rows [16w, 16w + 16) of K and of V with two 1 KB
    // buffer_load ... lds each; lane l of instruction j brings row 16w + 8j + l / 8, chunk position
    // l % 8 (the global chunk that the swizzle puts there). Loads past the buffer range write zeros.
    uint32_t dma_k_off[2], dma_v_off[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t row = static_cast<uint32_t>(16 * wave + 8 * j + (lane >> 3));
        const uint32_t pos = static_cast<uint32_t>(lane & 7);
        dma_k_off[j] = row * k_row_bytes + 16 * (pos ^ ((row >> 1) & 7));
        dma_v_off[j] = row * v_row_bytes + 16 * (pos ^ (((row >> 1) & 1) << 2));
    }
    // Issues the loads of KV tile kt into buffer kt % 3 (rows past the end load zeros): 16 bytes
    // a lane straight into LDS (buffer_load ... lds; M0 holds the LDS address of the wave's 1 KB).
    // The whole byte offset goes in the lane's offset register: the buffer range check covers that
    // register (and the instruction offset) but not the scalar offset, so rows past the end read
    // zeros instead of whatever memory follows the tensor.
    // Written as inline asm: the compiler does not see LDS writes in flight that it cannot tell
    // apart from the buffers being read, and would otherwise wait for these loads before every
    // LDS read, which makes them synchronous. Their completion is waited for explicitly (vmcnt)
    // before each barrier. They have no destination registers; the asm reads its operands at issue.
    auto dma = [&](int kt) SA_INLINE {
        const int b = kt % kStages;
        const uint32_t k_tile_off = static_cast<uint32_t>(kt * kKeyTile) * k_row_bytes;
        const uint32_t v_tile_off = static_cast<uint32_t>(kt * kKeyTile) * v_row_bytes;
        if constexpr (kPoisonLds) {
            // NaN into the 16 bytes each load below will write (lane l: byte 16 l of the wave's
            // 1 KB), complete before the loads are issued.
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                *reinterpret_cast<bf16x8*>(&k_lds[b][(16 * wave + 8 * j) * 64 + 8 * lane]) = nan_bf16x8();
                *reinterpret_cast<bf16x8*>(&v_lds[b][(16 * wave + 8 * j) * 64 + 8 * lane]) = nan_bf16x8();
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t k_dst = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                (__attribute__((address_space(3))) void*)&k_lds[b][(16 * wave + 8 * j) * 64]));
            const uint32_t v_dst = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                (__attribute__((address_space(3))) void*)&v_lds[b][(16 * wave + 8 * j) * 64]));
            asm volatile(
                "s_mov_b32 m0, %0\n\t"
                "s_nop 0\n\t"
                "buffer_load_dwordx4 %1, %2, 0 offen lds"
                :
                : "s"(k_dst), "v"(dma_k_off[j] + k_tile_off), "s"(krs)
                : "memory", "m0");
            asm volatile(
                "s_mov_b32 m0, %0\n\t"
                "s_nop 0\n\t"
                "buffer_load_dwordx4 %1, %2, 0 offen lds"
                :
                : "s"(v_dst), "v"(dma_v_off[j] + v_tile_off), "s"(vrs)
                : "memory", "m0");
        }
    };
    // Every tile kt passes one barrier, B_kt, somewhere after the wave has finished reading tile
    // kt - 1 and before it reads anything of tile kt + 1. Before B_kt the wave waits for its own
    // loads of tile kt + 1 (the only ones in flight); after B_kt those of every wave have landed, and
    // the wave issues the loads of tile kt + 2 into the buffer of tile kt - 1, which nobody reads any
    // more. The running-max tiles put B_kt first; the pipelined tiles put it half-way, so the first
    // K operands of tile kt + 1 are read during tile kt.
    auto tile_barrier = [&](int kt) SA_INLINE {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt unconstrained
        __syncthreads();
        dma(kt + 2);
    };

    // Transpose-read addressing for the V^T operand (16-lane group a = lane / 16): lane
    // 16a + L points at tile row 4 * (a / 2) + L / 4 (+ 8 for k-slots 4..7) and column
    // 16 * (a % 2) + 4 * (L % 4) of the 32-column block n; it receives d = 32n + (lane % 32).
    const int tr_row = 4 * half + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    float m[2], dsum[2];
    f32x16 acc[2][2];

    // S^T register r of block mb (32 keys) holds key key0 + 32 mb + 8 (r / 4) + 4 half + r % 4 of
    // the lane's query row; P^T k-step u = 2 mb + r / 8 takes registers 8 (u % 2) .. + 7 of it.
    // V^T k-step u, d-block n: lane reads row 16u + tr_row (and + 8), chunk 4n + tr_col / 8 of it,
    // 8 bytes at tr_col % 8; the swizzle of those rows is ((tr_row >> 1) & 1) << 2.
    const int v_lane_off = tr_row * 64 + (tr_col & 7) + 8 * ((tr_col >> 3) ^ (((tr_row >> 1) & 1) << 2));
    auto v_step = [&](const __bf16* vt, int u, bf16x8 (&vo)[2]) SA_INLINE {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            // chunk 4n + x with x < 4: the swizzle (0 or 4) only flips n's bit, folded into v_lane_off
            const __bf16* vrow = &vt[16 * u * 64 + (v_lane_off ^ (32 * n))];
            const bf16x4 lo4 = lds_read_tr4(vrow);
            const bf16x4 hi4 = lds_read_tr4(vrow + 8 * 64);
            vo[n] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    // K rows 32 mb + col, chunk 2 ks + half at position (2 ks + half) ^ ((col >> 1) & 7).
    int k_lane_off[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) k_lane_off[ks] = col * 64 + 8 * ((2 * ks + half) ^ ((col >> 1) & 7));
    auto k_half = [&](const __bf16* kt_, int mb, bf16x8 (&ko)[4]) SA_INLINE {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            ko[ks] = *reinterpret_cast<const bf16x8*>(&kt_[32 * mb * 64 + k_lane_off[ks]]);
    };

    // Exponentials exp2(c2 s - m) of registers [r0, r0 + nr) of one S^T block into P^T operands,
    // with the row sum taken on the rounded values (v_dot2 with (1, 1)) so numerator and
    // denominator use the same P: the rounding of a dominant weight then cancels in O / d (a sum of
    // the unrounded fp32 terms measured 0.023 max-abs against 0.015 on rows whose logits grow 8x
    // past their first keys). On the zero reference (m = 0) this is one multiply per score.
    auto exp_regs = [&](const f32x16& sb, float neg_m, bool zero_ref, bf16x8 (&pp)[4], int mb, int r0, int nr,
                        float& pa, float& pb, bool row_sum = true) SA_INLINE {
#pragma unroll
        for (int r = r0; r < r0 + nr; r += 2) {
            bf16x2 pr;
            pr[0] = (__bf16)exp2_fast(zero_ref ? sb[r] * c2 : fmaf(sb[r], c2, neg_m));
            pr[1] = (__bf16)exp2_fast(zero_ref ? sb[r + 1] * c2 : fmaf(sb[r + 1], c2, neg_m));
            pp[2 * mb + (r >> 3)][r & 7] = pr[0];
            pp[2 * mb + (r >> 3)][(r & 7) + 1] = pr[1];
            if (row_sum) {
                if (r & 2) pb = sum_bf16x2(pr, pb); else pa = sum_bf16x2(pr, pa);
            }
        }
    };
    // Causal / sequence-end mask of one S^T block: compare the compile-time key offset against
    // one per-row relative limit.
    auto mask_block = [&](f32x16& sb, int cb, int mb, int key0) SA_INLINE {
        const int limit = p.causal ? min(k_len, pos[cb] + offset + 1) : k_len;
        const int rel = limit - key0 - 4 * half;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (32 * mb + 8 * (r >> 2) + (r & 3) >= rel) sb[r] = kNegInf;
    };
    auto wave_zero_ref = [&]() { return __all(m[0] == 0.0f && m[1] == 0.0f); };

    // A plain tile (general reference, or zero reference with masking): all S^T first, then the
    // softmax of each column block, then O^T += V^T . P^T.
    auto plain_tile = [&](int kt, auto masked_tag, auto fast_tag, auto allow_switch_tag) SA_INLINE {
        constexpr bool kMasked = decltype(masked_tag)::value;
        constexpr bool kZero = decltype(fast_tag)::value;
        constexpr bool kSwitch = decltype(allow_switch_tag)::value;
        const int buf = kt % kStages;
        const int key0 = kt * kKeyTile;
        tile_barrier(kt);
        __builtin_amdgcn_sched_barrier(0);
        f32x16 s[2][2];
        {
            bf16x8 ko[2][4];
            k_half(k_lds[buf], 0, ko[0]);
            k_half(k_lds[buf], 1, ko[1]);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    s[cb][mb] = mfma32x32x16(ko[mb][0], q_op[cb][0], zero_f32x16());
#pragma unroll
                    for (int ks = 1; ks < 4; ++ks) s[cb][mb] = mfma32x32x16(ko[mb][ks], q_op[cb][ks], s[cb][mb]);
                }
        }
        bf16x8 pp[2][4];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            if constexpr (kMasked) {
                mask_block(s[cb][0], cb, 0, key0);
                mask_block(s[cb][1], cb, 1, key0);
            }
            float neg_m = 0.0f;
            if constexpr (!kZero) {
                // Running max with lazy rescaling.
                float bmax = kNegInf;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) bmax = fmaxf(bmax, s[cb][mb][r]);
                bmax = max_xor32(bmax) * c2;  // scale > 0, so the max commutes with it
                if (__any(bmax > m[cb] + kRescaleSlack)) {
                    const float m_new = fmaxf(m[cb], bmax);
                    const float alpha = exp2_fast(m[cb] - (m_new == kNegInf ? 0.0f : m_new));
                    dsum[cb] *= alpha;
#pragma unroll
                    for (int n = 0; n < 2; ++n) acc[cb][n] *= alpha;
                    m[cb] = m_new;
                }
                neg_m = m[cb] == kNegInf ? 0.0f : -m[cb];
            }
            float pa = 0.0f, pb = 0.0f;
            exp_regs(s[cb][0], neg_m, kZero, pp[cb], 0, 0, 16, pa, pb);
            exp_regs(s[cb][1], neg_m, kZero, pp[cb], 1, 0, 16, pa, pb);
            dsum[cb] += pa + pb;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            bf16x8 vo[2];
            v_step(v_lds[buf], u, vo);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int n = 0; n < 2; ++n) acc[cb][n] = mfma32x32x16(vo[n], pp[cb][u], acc[cb][n]);
        }
        if constexpr (kSwitch) {
            // Rows whose running max is moderate move to the zero reference (exact up to one
            // rounding of O and d), after this tile's P has been accumulated relative to the old
            // reference.
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                if (m[cb] != 0.0f && m[cb] >= -kZeroRefLimit && m[cb] <= kZeroRefLimit) {
                    const float alpha = exp2_fast(m[cb]);
                    dsum[cb] *= alpha;
#pragma unroll
                    for (int n = 0; n < 2; ++n) acc[cb][n] *= alpha;
                    m[cb] = 0.0f;
                }
            }
        }
    };

    // Unmasked tiles with every row of the wave on the zero reference, software-pipelined across
    // tiles. Per tile there are four S^T blocks S_cb,mb (column block cb, key half mb: 4 MFMAs
    // each), eight half-block exponential groups E_cb,mb,h (registers 8h..8h+7 of S_cb,mb; they give
    // the P^T operand of k-step u = 2 mb + h) and four PV k-steps PV(u) (O^T += V^T . P^T for both
    // column blocks: 4 MFMAs each). Every slot pairs four MFMAs with one exponential group, and
    // every MFMA or exponential consumes what an earlier slot produced:
    //   t1: S00      | E11a (previous tile)     t5: S01 | E10a
    //   t2: S10      | E11b (previous tile)     t6: PV0 | E10b
    //   t3: PV2 (previous tile) | E00a          t7: S11 | E01a
    //   t4: PV3 (previous tile) | E00b          t8: PV1 | E01b
    // So S11's exponentials and the last two k-steps carry into the next tile: S11, the P^T of E01
    // and the V^T operands of k-steps 2 and 3 stay in registers across the barrier (V^T is read
    // from LDS before it), and every LDS read of a tile still happens between its two barriers, so
    // double buffering suffices. t1 issues its exponentials first: they cover the K reads that
    // follow the barrier. The first tile of a run has no carried work; drain_fast finishes the
    // last one.
    // Row sums come from the matrix core, on exactly the bf16 P the PV products use: a P^T operand
    // (16 keys x 32 rows), read as the B operand of v_mfma_f32_16x16x32_bf16, holds in its 32 k-slots
    // keys 0-7 and 8-15 of rows n and n + 16 (n = lane % 16); an A operand of ones and zeros that
    // picks the row-n slots for output rows 0-7 and the row-(n + 16) slots for rows 8-15 gives
    // the 16-key sums of all 32 rows. One such MFMA per P^T operand, in the slot after the one that
    // made the operand, accumulates into rsum[cb]; lane l ends up with the sum of row
    // (l % 16) + 16 (l / 32) in all four registers.
    f32x16 fs00, fs10, fs01, fs11;
    bf16x8 fp0[4], fp1[4];  // P^T operands of column blocks 0 and 1, by k-step
    bf16x8 vcarry[2][2];    // V^T operands of k-steps 2 and 3 (by d-block n) of the previous tile
    f32x4 rsum[2];
    bf16x8 rsum_sel;
    bf16x8 kpre[4];  // K operands of the first key half of the next tile
    {
        const __bf16 one = (((lane >> 4) & 1) == ((lane & 15) >> 3)) ? (__bf16)1.0f : (__bf16)0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) rsum_sel[e] = one;
    }
    float no_sum = 0.0f;
#define SA_PIN_ACC() asm volatile("" : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]))
#define SA_SLOT_END() __builtin_amdgcn_sched_barrier(0)
#define SA_MFMA_FIRST(n_valu)                                            \
    do {                                                                 \
        for (int i_ = 0; i_ < 4; ++i_) {                                 \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           \
            __builtin_amdgcn_sched_group_barrier(0x002, (n_valu), 0);    \
        }                                                                \
    } while (0)
#define SA_VALU_FIRST(n_valu)                                            \
    do {                                                                 \
        for (int i_ = 0; i_ < 4; ++i_) {                                 \
            __builtin_amdgcn_sched_group_barrier(0x002, (n_valu), 0);    \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           \
        }                                                                \
    } while (0)
    auto s_block = [&](f32x16& sb, const bf16x8 (&ko)[4], int cb) SA_INLINE {
        sb = mfma32x32x16(ko[0], q_op[cb][0], zero_f32x16());
#pragma unroll
        for (int ks = 1; ks < 4; ++ks) sb = mfma32x32x16(ko[ks], q_op[cb][ks], sb);
    };
    auto pv_step = [&](const bf16x8 (&vo)[2], int u) SA_INLINE {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[j >> 1][j & 1] = mfma32x32x16(vo[j & 1], (j >> 1) ? fp1[u] : fp0[u], acc[j >> 1][j & 1]);
    };
    auto row_sum = [&](int cb, const bf16x8& pt) SA_INLINE { rsum[cb] = mfma16x16x32(rsum_sel, pt, rsum[cb]); };
    // buf_tag: the tile's LDS buffer (kt % 3) as a compile-time constant, or -1 to compute it. With a
    // constant buffer every LDS read folds the buffer into its immediate offset; computed, each
    // read's lane address needs a vector add per tile.
    auto fast_tile = [&](int kt, auto carry_tag, auto buf_tag) SA_INLINE {
        constexpr bool kCarry = decltype(carry_tag)::value;
        constexpr int kBuf = decltype(buf_tag)::value;
        const int buf = kBuf >= 0 ? kBuf : kt % kStages;
        const int next_buf = kBuf >= 0 ? (kBuf + 1) % kStages : (kt + 1) % kStages;
        const __bf16* kt_lds = k_lds[buf];
        const __bf16* vt_lds = v_lds[buf];
        bf16x8 k1[4], va[2], vb[2];
        // K of the first key half: read during the previous pipelined tile, else now.
        if constexpr (!kCarry) k_half(kt_lds, 0, kpre);
        __builtin_amdgcn_sched_barrier(0);
        // t1: S00 | E11a (previous tile)
        if constexpr (kCarry) exp_regs(fs11, 0.0f, true, fp1, 1, 0, 8, no_sum, no_sum, false);
        s_block(fs00, kpre, 0);
        if constexpr (kCarry) {
            row_sum(0, fp0[3]);
            SA_VALU_FIRST(5);
            asm volatile("" : "+v"(fp1[2]), "+v"(rsum[0]));
        }
        asm volatile("" : "+v"(fs00));
        SA_SLOT_END();
        // t2: S10 | E11b (previous tile)
        s_block(fs10, kpre, 1);
        if constexpr (kCarry) {
            exp_regs(fs11, 0.0f, true, fp1, 1, 8, 8, no_sum, no_sum, false);
            row_sum(1, fp1[2]);
            SA_MFMA_FIRST(5);
            asm volatile("" : "+v"(fp1[3]), "+v"(rsum[1]));
        }
        asm volatile("" : "+v"(fs10));
        SA_SLOT_END();
        // t3: PV2 (previous tile) | E00a; K of the second key half
        k_half(kt_lds, 1, k1);
        if constexpr (kCarry) {
            pv_step(vcarry[0], 2);
            row_sum(1, fp1[3]);
        }
        exp_regs(fs00, 0.0f, true, fp0, 0, 0, 8, no_sum, no_sum, false);
        if constexpr (kCarry) {
            SA_MFMA_FIRST(5);
            SA_PIN_ACC();
            asm volatile("" : "+v"(rsum[1]));
        }
        asm volatile("" : "+v"(fp0[0]));
        SA_SLOT_END();
        // t4: PV3 (previous tile) | E00b; V^T of k-step 0
        v_step(vt_lds, 0, va);
        if constexpr (kCarry) pv_step(vcarry[1], 3);
        row_sum(0, fp0[0]);
        exp_regs(fs00, 0.0f, true, fp0, 0, 8, 8, no_sum, no_sum, false);
        if constexpr (kCarry) {
            SA_MFMA_FIRST(5);
            SA_PIN_ACC();
        }
        asm volatile("" : "+v"(fp0[1]), "+v"(rsum[0]));
        SA_SLOT_END();
        tile_barrier(kt);
        // t5: S01 | E10a
        s_block(fs01, k1, 0);
        row_sum(0, fp0[1]);
        exp_regs(fs10, 0.0f, true, fp1, 0, 0, 8, no_sum, no_sum, false);
        SA_MFMA_FIRST(5);
        asm volatile("" : "+v"(fs01), "+v"(fp1[0]), "+v"(rsum[0]));
        SA_SLOT_END();
        // t6: PV0 | E10b; V^T of k-step 1
        v_step(vt_lds, 1, vb);
        pv_step(va, 0);
        row_sum(1, fp1[0]);
        exp_regs(fs10, 0.0f, true, fp1, 0, 8, 8, no_sum, no_sum, false);
        SA_MFMA_FIRST(5);
        SA_PIN_ACC();
        asm volatile("" : "+v"(fp1[1]), "+v"(rsum[1]));
        SA_SLOT_END();
        // t7: S11 | E01a; V^T of k-step 2 (carried)
        v_step(vt_lds, 2, vcarry[0]);
        s_block(fs11, k1, 1);
        row_sum(1, fp1[1]);
        exp_regs(fs01, 0.0f, true, fp0, 1, 0, 8, no_sum, no_sum, false);
        SA_MFMA_FIRST(5);
        asm volatile("" : "+v"(fs11), "+v"(fp0[2]), "+v"(rsum[1]));
        SA_SLOT_END();
        // t8: PV1 | E01b; V^T of k-step 3 (carried); K of the next tile's first key half
        v_step(vt_lds, 3, vcarry[1]);
        k_half(k_lds[next_buf], 0, kpre);
        pv_step(vb, 1);
        row_sum(0, fp0[2]);
        exp_regs(fs01, 0.0f, true, fp0, 1, 8, 8, no_sum, no_sum, false);
        SA_MFMA_FIRST(5);
        SA_PIN_ACC();
        asm volatile("" : "+v"(fp0[3]), "+v"(rsum[0]));
        SA_SLOT_END();
    };
    // The carried work of the last pipelined tile: E11, then k-steps 2 and 3.
    auto drain_fast = [&]() SA_INLINE {
        exp_regs(fs11, 0.0f, true, fp1, 1, 0, 16, no_sum, no_sum, false);
        row_sum(0, fp0[3]);
        row_sum(1, fp1[2]);
        row_sum(1, fp1[3]);
        pv_step(vcarry[0], 2);
        pv_step(vcarry[1], 3);
        // Lane l holds the sum of row (l % 16) + 16 (l / 32); the lane of column col = l % 32 takes
        // it from lane (col % 16) + 32 (col / 16), keeping it in its half-0 share of d.
        const int src = (col & 15) + 32 * (col >> 4);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const float mine = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * src, __builtin_bit_cast(int, rsum[cb][0])));
            dsum[cb] += half == 0 ? mine : 0.0f;
        }
    };
#undef SA_PIN_ACC
#undef SA_SLOT_END
#undef SA_MFMA_FIRST
#undef SA_VALU_FIRST

    using False = std::integral_constant<bool, false>;
    using True = std::integral_constant<bool, true>;
    // All KV tiles of the work-group. With kAllowFast, rows move to the zero reference as soon as
    // their running max allows it, and a wave whose rows all have moved runs fast tiles.
    auto process = [&](auto allow_fast_tag) SA_INLINE {
        constexpr bool kAllowFast = decltype(allow_fast_tag)::value;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            // Sink fold: m starts at the head's sink, d at 1 (kept in the half-0 lane's share);
            // a split other than the first starts empty (m = -inf, d = 0). A row whose sink lies
            // in [-kZeroRefLimit, kZeroRefLimit] may start on the zero reference instead (m = 0,
            // d = 2^sink): the sink term alone gives the row a term >= 2^-kZeroRefLimit, the
            // condition the switch after a running-max tile checks, so even the first tile can
            // run without row maxima.
            m[cb] = carries_sink ? sink2[cb] : kNegInf;
            dsum[cb] = (half == 0 && m[cb] != kNegInf && !kMutateD0Zero) ? 1.0f : 0.0f;
            if (kAllowFast && m[cb] >= -kZeroRefLimit && m[cb] <= kZeroRefLimit) {
                dsum[cb] = (half == 0 && !kMutateD0Zero) ? exp2_fast(m[cb]) : 0.0f;
                m[cb] = 0.0f;
            }
#pragma unroll
            for (int n = 0; n < 2; ++n) acc[cb][n] = zero_f32x16();
        }
        if (kt_begin < kt_end) {
            dma(kt_begin);
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            __syncthreads();
            dma(kt_begin + 1);
        }
        const int unmasked_end = min(mask_from, kt_end);
        // Running-max tiles until every row of the wave is on the zero reference (with kAllowFast;
        // the rows switch as soon as their running max allows it), then pipelined zero-reference
        // tiles to the end, the masked ones (diagonal, sequence end) included. Every tile of either
        // kind ends with the same one barrier, so waves of one work-group may mix them.
        int kt = kt_begin;
        while (kt < kt_end && !(kAllowFast && wave_zero_ref())) {
            if (kt < unmasked_end)
                plain_tile(kt, False(), False(), allow_fast_tag);
            else
                plain_tile(kt, True(), False(), allow_fast_tag);
            ++kt;
        }
        if constexpr (kAllowFast) {
            if (kt < unmasked_end) {
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) rsum[cb] = zero_f32x4();
                using Computed = std::integral_constant<int, -1>;
                fast_tile(kt++, False(), Computed());
                // Up to buffer 0, then three tiles at a time with their buffers known at compile
                // time, then the remainder.
                for (; kt < unmasked_end && kt % kStages != 0; ++kt) fast_tile(kt, True(), Computed());
                for (; kt + kStages <= unmasked_end; kt += kStages) {
                    fast_tile(kt, True(), std::integral_constant<int, 0>());
                    fast_tile(kt + 1, True(), std::integral_constant<int, 1>());
                    fast_tile(kt + 2, True(), std::integral_constant<int, 2>());
                }
                for (; kt < unmasked_end; ++kt) fast_tile(kt, True(), Computed());
                drain_fast();
            }
            for (; kt < kt_end; ++kt) plain_tile(kt, True(), True(), False());
        }
        // The last two tiles' loads (past the end: zeros) must land before LDS is reused or
        // released.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    };

    // Zero-reference tiles leave p = exp2(s) unbounded above. If any row's d left the range where
    // that is safe (d > 2^64, or any non-finite d or O), the whole work-group starts again with
    // the running-max reference only; the decision is work-group wide because the waves share
    // the K/V tiles and their barriers.
    __shared__ int redo_general;
    process(True());
    bool bad = false;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        bad |= !(dsum[cb] <= kFastSumLimit);
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) bad |= !__builtin_isfinite(acc[cb][n][r]);
    }
    // Poisoned-LDS builds never start again: a NaN read from a poisoned buffer must reach the
    // output rather than be recomputed (they are run on inputs that need no second pass).
    if constexpr (kPoisonLds) bad = false;
    if (tid == 0) redo_general = 0;
    __syncthreads();
    if (__any(bad) && lane == 0) redo_general = 1;
    __syncthreads();
    if (redo_general) process(False());

    // Epilogue: out = acc / d. Lane holds d-channels 32n + 8 (r / 4) + 4 half + r % 4.
    // bf16 output goes through LDS: each wave writes its 64 rows x 64 d row-major into one of the
    // K/V buffers (free once every wave is past its last tile), then stores whole 128-byte rows,
    // eight lanes per row: the rows of one position's heads are adjacent in memory, so every store
    // instruction writes full lines instead of 16 bytes of 32 rows. 16-byte chunk c of row r sits
    // at c ^ (r & 7), its two 8-byte halves swapped when r & 8: the 8-byte writes of 16 rows and
    // the 16-byte reads of 8 rows then hit distinct banks.
    // Split-KV prefill writes the split's state instead: o = acc / d, m (natural log), d.
    if constexpr (!kSplit) {
        if (p.out_is_bf16) {
            if (redo_general) __syncthreads();  // the second pass ends without a barrier
            __bf16* stage = wave < kStages ? k_lds[wave] : v_lds[wave - kStages];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const float dtot = sum_xor32(dsum[cb]);
                const float inv = dtot > 0.0f ? 1.0f / dtot : 0.0f;
                const int row = cb * 32 + col;
#pragma unroll
                for (int n = 0; n < 2; ++n)
#pragma unroll
                    for (int quad = 0; quad < 4; ++quad) {
                        bf16x4 o;
#pragma unroll
                        for (int i = 0; i < 4; ++i) o[i] = (__bf16)(acc[cb][n][4 * quad + i] * inv);
                        *reinterpret_cast<bf16x4*>(
                            &stage[row * 64 + 8 * ((4 * n + quad) ^ (row & 7)) + 4 * (half ^ ((row >> 3) & 1))]) = o;
                    }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int row = 8 * j + (lane >> 3), c = lane & 7;
                bf16x8 o = *reinterpret_cast<const bf16x8*>(&stage[row * 64 + 8 * (c ^ (row & 7))]);
                if (j & 1) o = __builtin_shufflevector(o, o, 4, 5, 6, 7, 0, 1, 2, 3);  // row & 8: halves swapped
                const int r = wave * kRowsPerWave + row;
                const int rpos = first_pos + r / group;
                if (rpos >= q_len) continue;
                *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(p.out) +
                                           static_cast<int64_t>(q_start + rpos) * p.o_stride_tok +
                                           static_cast<int64_t>(g * group + r % group) * p.o_stride_head + 8 * c) = o;
            }
            return;
        }
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const float dtot = sum_xor32(dsum[cb]);
        if (!valid[cb]) continue;
        const float inv = dtot > 0.0f ? 1.0f / dtot : 0.0f;
        if constexpr (kSplit) {
            const int64_t row = (static_cast<int64_t>(q_start + pos[cb]) * p.num_q_heads + head[cb]) * p.num_splits + split;
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int quad = 0; quad < 4; ++quad) {
                    f32x4 o;
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = acc[cb][n][4 * quad + i] * inv;
                    *reinterpret_cast<f32x4*>(p.partial_o + row * kHeadDim + 32 * n + 8 * quad + 4 * half) = o;
                }
            if (half == 0) {
                p.partial_m[row] = dtot > 0.0f ? m[cb] * kLn2 : kNegInf;
                p.partial_d[row] = dtot;
            }
            continue;
        }
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
    for (int d = 0; d < kHeadDim; ++d) qv[d] = qrow[d];
    const float* kb = static_cast<const float*>(p.k) + static_cast<int64_t>(k_start) * p.k_stride_tok +
                      static_cast<int64_t>(g) * p.k_stride_head;
    const float* vb = static_cast<const float*>(p.v) + static_cast<int64_t>(k_start) * p.v_stride_tok +
                      static_cast<int64_t>(g) * p.v_stride_head;
    // Keys [j0, j1) folded into (m, dsum, acc) with the page's recurrence.
    float m, dsum;
    auto fold = [&](int j0, int j1) {
        for (int j = j0; j < j1; ++j) {
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
    };
    auto start = [&](bool with_sink) {
        m = with_sink ? p.sinks[head] : kNegInf;
        dsum = (m == kNegInf || kMutateD0Zero) ? 0.0f : 1.0f;
        for (int d = 0; d < kHeadDim; ++d) acc[d] = 0.0f;
    };
    if (p.partial_o != nullptr) {
        // Split-KV prefill: every split of this row in turn (boundaries as in the bf16 kernel).
        const int per = (k_len + p.num_splits - 1) / p.num_splits;
        const int split_keys = (per + 63) / 64 * 64;
        for (int sp = 0; sp < p.num_splits; ++sp) {
            const int lo = min(sp * split_keys, k_len);
            const int hi = min(lo + split_keys, key_end);
            start(sp == 0 || kMutateSinkEveryChunk);
            fold(lo, hi);
            const int64_t row = (static_cast<int64_t>(tok) * p.num_q_heads + head) * p.num_splits + sp;
            const float inv = dsum > 0.0f ? 1.0f / dsum : 0.0f;
            for (int d = 0; d < kHeadDim; ++d) p.partial_o[row * kHeadDim + d] = acc[d] * inv;
            p.partial_m[row] = dsum > 0.0f ? m : kNegInf;
            p.partial_d[row] = dsum;
        }
        return;
    }
    start(true);
    fold(0, key_end);
    const float inv = dsum > 0.0f ? 1.0f / dsum : 0.0f;
    float* orow = static_cast<float*>(p.out) + static_cast<int64_t>(tok) * p.o_stride_tok +
                  static_cast<int64_t>(head) * p.o_stride_head;
    for (int d = 0; d < kHeadDim; ++d) orow[d] = acc[d] * inv;
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream) {
    const Launch l = plan_prefill_bf16(p);
    if (l.grid > kMaxGrid) return hipErrorInvalidConfiguration;
    if (p.partial_o != nullptr)
        prefill_bf16_kernel<true><<<dim3(static_cast<unsigned>(l.grid)), dim3(l.block), 0, stream>>>(p);
    else
        prefill_bf16_kernel<false><<<dim3(static_cast<unsigned>(l.grid)), dim3(l.block), 0, stream>>>(p);
    return hipGetLastError();
}

hipError_t launch_prefill_f32(const PrefillParams& p, hipStream_t stream) {
    const Launch l = plan_prefill_f32(p);
    if (l.grid > kMaxGrid) return hipErrorInvalidConfiguration;
    prefill_f32_kernel<<<dim3(static_cast<unsigned>(l.grid)), dim3(l.block), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace sinkattn
