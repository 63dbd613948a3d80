// Launch plans: which kernel instance, grid and work-group size every attention launcher uses, as
// plain host code. The launchers in the .hip files launch exactly what these functions return; the
// C-ABI reports them without launching (sinkattn_plan_*), and a host-only build of api.cpp checks
// them on the CPU.
#pragma once

#include <stdint.h>
#include <stdio.h>

#include "launch.h"

namespace sinkattn {

// Compute units of an MI355X / MI350X (gfx950).
constexpr int64_t kComputeUnits = 256;

// Split-KV decode (decode_split.hip): four waves per KV head of a work-group.
constexpr int kSplitWaves = 4;
constexpr int kSplitThreads = kSplitWaves * 64;

// Causal prefill (prefill.hip): four waves, 64 query rows each.
constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kRowsPerWave = 64;
constexpr int kRowsPerTile = kPfWaves * kRowsPerWave;  // 256 query rows per work-group

// Chunk merge (decode_merge.hip): four waves; four rows per wave from kRowsForX4 rows on.
constexpr int kMergeWaves = 4;
constexpr int64_t kRowsForX4 = 8192;
constexpr int kMergeX4MaxChunks = 16;

// Reference fp32 kernels: one thread per (token, head) row or per chunk state.
constexpr int kF32Threads = 256;

// One launch: the kernel's name as a profiler prints it (without namespace and parameter list),
// its grid in work-groups and its work-group size in threads.
struct Launch {
    char kernel[96];
    int64_t grid;
    int32_t block;
};

inline Launch make_launch(const char* kernel, int64_t grid, int32_t block) {
    Launch l{};
    snprintf(l.kernel, sizeof(l.kernel), "%s", kernel);
    l.grid = grid;
    l.block = block;
    return l;
}

inline const char* bool_name(bool x) { return x ? "true" : "false"; }

// ---------------------------------------------------------------------------- split-KV decode
// Adjacent KV heads are grouped per work-group where their slices of a cache row are adjacent
// (token-major caches): the wider the contiguous piece of every row a work-group reads, the closer
// the stream comes to the copy rate (measured on MI355X: one head 345 us, two 307 us, four 283 us
// on 32 sequences of 16K-32K keys). Four heads (512 bytes of every row, 1024 threads, one
// work-group per CU) when that still gives at least two rounds of work-groups; two heads when the
// paired grid gives every compute unit a work-group; otherwise one. With one column tile (G x T <=
// 16 query rows per KV head) the four waves of a KV head split the keys of each block (key split);
// with more, each wave folds one column tile over all keys.
struct DecodeShape {
    int heads;       // KV heads per work-group: 1, 2 or 4
    bool key_split;  // the waves of a KV head split the keys (G x T <= 16)
    bool private_staging;  // each wave stages only its own keys' rows, no barrier per block
    int64_t groups;  // work-groups in the grid
    int block;       // threads per work-group
};

inline DecodeShape decode_shape(const DecodeSplitParams& p) {
    const bool adjacent = p.k_stride_head == kHeadDim && p.v_stride_head == kHeadDim;
    const int64_t paired = static_cast<int64_t>(p.batch) * (p.num_kv_heads / 2) * p.num_chunks;
    const int64_t quad = static_cast<int64_t>(p.batch) * (p.num_kv_heads / 4) * p.num_chunks;
    const int columns = p.num_q_heads / p.num_kv_heads * p.q_len;
    DecodeShape s{};
    s.key_split = columns <= 16;
    if (p.num_kv_heads % 4 == 0 && adjacent && quad >= 2 * kComputeUnits) {
        s.heads = 4;
        s.groups = quad;
    } else if (p.num_kv_heads % 2 == 0 && adjacent && paired >= kComputeUnits) {
        s.heads = 2;
        s.groups = paired;
    } else {
        s.heads = 1;
        s.groups = static_cast<int64_t>(p.batch) * p.num_kv_heads * p.num_chunks;
    }
    s.block = s.heads * kSplitThreads;
    // Private staging where it was measured faster: pairs of KV heads, key split, a single round of
    // work-groups (8 x 8192 keys: split + merge 26.0 vs 27.1 us); the multi-round grids of four
    // heads were 7-8% slower with it.
    s.private_staging = s.heads == 2 && s.key_split && s.groups <= kComputeUnits;
    return s;
}

// The single launch (split and merge together) pays only when the split grid has at most one
// work-group per compute unit: on a longer grid every work-group that finishes early holds its
// compute unit through the arrival count and, for the last one, the merge, while split then merge
// does not.
inline bool decode_fused_fits_one_round(const DecodeSplitParams& p) {
    return decode_shape(p).groups <= kComputeUnits;
}

inline Launch plan_decode_split_bf16(const DecodeSplitParams& p, bool fused) {
    const DecodeShape s = decode_shape(p);
    char name[96];
    snprintf(name, sizeof(name), "decode_split_bf16_kernel<%d, %s, %s, %s>", s.heads, bool_name(fused),
             bool_name(s.key_split), bool_name(s.private_staging));
    return make_launch(name, s.groups, s.block);
}

inline Launch plan_decode_split_f32(const DecodeSplitParams& p) {
    const int64_t states = static_cast<int64_t>(p.batch) * p.q_len * p.num_q_heads * p.num_chunks;
    return make_launch("decode_split_f32_kernel", (states + kF32Threads - 1) / kF32Threads, kF32Threads);
}

// ---------------------------------------------------------------------------- chunk merge
inline bool merge_four_rows_per_wave(const DecodeMergeParams& p) {
    return static_cast<int64_t>(p.batch) * p.num_q_heads >= kRowsForX4 && p.num_chunks <= kMergeX4MaxChunks;
}

inline Launch plan_decode_merge(const DecodeMergeParams& p) {
    const int64_t rows = static_cast<int64_t>(p.batch) * p.num_q_heads;
    if (merge_four_rows_per_wave(p))
        return make_launch("decode_merge_x4_kernel", (rows + 4 * kMergeWaves - 1) / (4 * kMergeWaves),
                           kMergeWaves * 64);
    return make_launch("decode_merge_kernel", (rows + kMergeWaves - 1) / kMergeWaves, kMergeWaves * 64);
}

// ---------------------------------------------------------------------------- prefill
// One work-group per (query tile, KV head[, key split]); a query tile is kRowsPerTile / G
// consecutive positions of one sequence for the G query heads of the KV head. The grid is an upper
// bound taken without reading cu_seqlens: each sequence adds at most one partial tile beyond
// ceil(Tq / positions per tile); work-groups past the last tile exit at once.
struct PrefillShape {
    int positions_per_tile;
    int64_t tiles;  // upper bound on query tiles
    int64_t blocks;
    bool split;     // per-split states (sinkattn_prefill_split)
};

inline PrefillShape prefill_shape(const PrefillParams& p) {
    PrefillShape s{};
    const int group = p.num_q_heads / p.num_kv_heads;
    s.positions_per_tile = kRowsPerTile / group;
    s.tiles = (p.total_q + s.positions_per_tile - 1) / s.positions_per_tile + p.num_seqs;
    s.split = p.partial_o != nullptr;
    s.blocks = s.tiles * p.num_kv_heads * (s.split ? p.num_splits : 1);
    return s;
}

inline Launch plan_prefill_bf16(const PrefillParams& p) {
    const PrefillShape s = prefill_shape(p);
    return make_launch(s.split ? "prefill_bf16_kernel<true>" : "prefill_bf16_kernel<false>", s.blocks, kPfThreads);
}

inline Launch plan_prefill_f32(const PrefillParams& p) {
    const int64_t rows = p.total_q * p.num_q_heads;
    return make_launch("prefill_f32_kernel", (rows + kF32Threads - 1) / kF32Threads, kF32Threads);
}

// Grids of 2^31 work-groups or more cannot be launched.
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;

}  // namespace sinkattn
