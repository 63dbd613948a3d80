// Linear layer with a bias folded into the matrix-core accumulators (gfx950):
//   Y[M, N] = X[M, K] W[N, K]^T + bias[N], in bf16, or in FP8 (OCP E4M3) with 128 x 128 block scaling.
//
// Source: "GPT-OSS on Day 0" (Perplexity). Section "GPT-OSS on Hopper" picks FP8 with 128x128 block
// scaling and a bias term for the GEMM kernels; section "Kernels for GPT-OSS" adds the bias by
// starting the accumulator registers at bias values loaded from memory once per output block. Here
// every 32x32 accumulator block starts at the bias: a lane's 16 accumulators share one output
// column (the MFMA C layout), so the bias costs one load per lane and block and no epilogue pass.
//
// Work-group: a 128 x 128 output tile, four waves of 64 x 64 (2 x 2 blocks of
// v_mfma_f32_32x32x16_bf16, or of v_mfma_scale_f32_32x32x64_f8f6f4 with unit E8M0 scales for FP8).
// Each K step stages 128 bytes of every A and B row (64 bf16 or 128 FP8 values = one scale block)
// in double-buffered LDS tiles of pitch 144 bytes (16-byte reads of 16 consecutive rows hit disjoint
// banks); the next step's loads are in flight while the current one is multiplied. FP8: each
// 128-wide k block is multiplied into a temporary accumulator, then added to the running one times
// scale_x[row, kb] * scale_w[column block, kb] (rows' scales staged in LDS with the tile).
// Tiles are spread XCD-aware: each XCD takes a contiguous range of tile indices, walked in groups of
// 8 tile-rows so the X and W panels a group shares stay in that XCD's L2.

#include "device_common.h"
#include "launch_ops.h"

namespace sinkattn {
namespace {

constexpr int kGemmThreads = 256;
constexpr int kTileN = 128;
constexpr int kStepBytes = 128;    // bytes of each row staged per K step
constexpr int kRowPitch = 144;     // LDS row pitch in bytes
constexpr int kGroupRows = 8;      // tile-rows per group in the tile order
constexpr int kGemmBM = 2;         // 32-row blocks per wave in M: tiles of 128 x 128 (256 x 128 measured slower)

typedef int i32x8 __attribute__((ext_vector_type(8)));

// kBM 32-row blocks per wave in M (two waves in M, two in N): tile (64 kBM) x 128. A step stages
// 8 sixteen-byte pieces per tile row: 2 kBM pieces of A and 4 of B per thread.
template <int kBM>
struct GemmStage {
    i32x4 a[2 * kBM];
    i32x4 b[4];
    float sx;  // FP8: the scale of tile row tid (threads below the tile's row count)
};

template <bool kFp8, int kBM>
__global__ __launch_bounds__(kGemmThreads, kBM == 2 ? 2 : 1) void gemm_bias_kernel(GemmParams p) {
    constexpr int kTileM = 64 * kBM;
    __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][kTileM][kRowPitch];
    __shared__ __attribute__((aligned(16))) uint8_t b_lds[2][kTileN][kRowPitch];
    __shared__ __attribute__((aligned(16))) float sx_lds[2][kTileM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, h = lane >> 5;

    // Tile order: contiguous ranges per XCD (work-groups go round-robin over the 8 XCDs), grouped.
    const int tiles_m = (p.m + kTileM - 1) / kTileM;
    const int tiles_n = (p.n + kTileN - 1) / kTileN;
    const int tiles = tiles_m * tiles_n;
    int t = blockIdx.x;
    if (tiles % 8 == 0) t = (t % 8) * (tiles / 8) + t / 8;
    const int per_group = kGroupRows * tiles_n;
    const int first_m = (t / per_group) * kGroupRows;
    const int group_rows = tiles_m - first_m < kGroupRows ? tiles_m - first_m : kGroupRows;
    const int tm = first_m + (t % per_group) % group_rows;
    const int tn = (t % per_group) / group_rows;
    const int m0 = tm * kTileM, n0 = tn * kTileN;

    // Operand slices of this work-group; rows past M or N load as zeros (buffer range).
    const int es = kFp8 ? 1 : 2;
    const int rows_a = p.m - m0 < kTileM ? p.m - m0 : kTileM;
    const int rows_b = p.n - n0 < kTileN ? p.n - n0 : kTileN;
    const uint32_t lda = static_cast<uint32_t>(p.ldx * es), ldb = static_cast<uint32_t>(p.ldw * es);
    const __amdgpu_buffer_rsrc_t ars =
        make_buffer(static_cast<const uint8_t*>(p.x) + static_cast<int64_t>(m0) * lda, rows_a * lda);
    const __amdgpu_buffer_rsrc_t brs =
        make_buffer(static_cast<const uint8_t*>(p.w) + static_cast<int64_t>(n0) * ldb, rows_b * ldb);

    // Accumulators start at the bias of their column (lane column r32 of each 32x32 block).
    f32x16 acc[kBM][2];
#pragma unroll
    for (int bn = 0; bn < 2; ++bn) {
        const int n = n0 + 64 * wn + 32 * bn + r32;
        const float b = p.bias != nullptr && n < p.n ? p.bias[n] : 0.0f;
#pragma unroll
        for (int bm = 0; bm < kBM; ++bm)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[bm][bn][i] = b;
    }

    // Thread piece j: row (tid + 256 j) / 8, 16-byte segment (tid + 256 j) % 8 of the step's bytes.
    auto stage_load = [&](GemmStage<kBM>& s, int step) {
        const uint32_t kb = static_cast<uint32_t>(step) * kStepBytes;
#pragma unroll
        for (int j = 0; j < 2 * kBM; ++j) {
            const int piece = tid + kGemmThreads * j;
            const uint32_t row = piece >> 3, seg = piece & 7;
            s.a[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, row * lda + kb + 16 * seg, 0, 0));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int piece = tid + kGemmThreads * j;
            const uint32_t row = piece >> 3, seg = piece & 7;
            s.b[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(brs, row * ldb + kb + 16 * seg, 0, 0));
        }
        if constexpr (kFp8) {
            const int row = m0 + tid;
            s.sx = tid < kTileM && row < p.m ? p.scale_x[row * p.sx_stride_m + step * p.sx_stride_kb] : 0.0f;
        }
    };
    auto stage_store = [&](const GemmStage<kBM>& s, int buf) {
#pragma unroll
        for (int j = 0; j < 2 * kBM; ++j) {
            const int piece = tid + kGemmThreads * j;
            *reinterpret_cast<i32x4*>(&a_lds[buf][piece >> 3][16 * (piece & 7)]) = s.a[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int piece = tid + kGemmThreads * j;
            *reinterpret_cast<i32x4*>(&b_lds[buf][piece >> 3][16 * (piece & 7)]) = s.b[j];
        }
        if constexpr (kFp8)
            if (tid < kTileM) sx_lds[buf][tid] = s.sx;
    };
    auto compute = [&](int buf, int step) {
        const uint8_t* arow[kBM];
        const uint8_t* brow[2];
#pragma unroll
        for (int q = 0; q < kBM; ++q) arow[q] = &a_lds[buf][32 * kBM * wm + 32 * q + r32][0];
#pragma unroll
        for (int q = 0; q < 2; ++q) brow[q] = &b_lds[buf][64 * wn + 32 * q + r32][0];
        if constexpr (!kFp8) {
            // Four k slices of 16 bf16; lane half h takes k 8h .. 8h + 7 of each slice.
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf16x8 av[kBM], bv[2];
#pragma unroll
                for (int q = 0; q < kBM; ++q) av[q] = *reinterpret_cast<const bf16x8*>(arow[q] + 32 * kk + 16 * h);
#pragma unroll
                for (int q = 0; q < 2; ++q) bv[q] = *reinterpret_cast<const bf16x8*>(brow[q] + 32 * kk + 16 * h);
#pragma unroll
                for (int bm = 0; bm < kBM; ++bm)
#pragma unroll
                    for (int bn = 0; bn < 2; ++bn) acc[bm][bn] = mfma32x32x16(av[bm], bv[bn], acc[bm][bn]);
            }
        } else {
            // Two k slices of 64 FP8; lane half h takes bytes 32h .. 32h + 31 of each slice (the
            // same bytes for A and B, so the product pairs equal k whatever order the unit uses).
            // Each block's two products go into a temporary that is promoted at once:
            // acc += part * scale_x[row] * scale_w (one weight scale per 128-column tile).
            const float sw = p.scale_w[static_cast<int64_t>(tn) * p.sw_stride_nb + step * p.sw_stride_kb];
            i32x8 bv[2][2];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const i32x4 b0 = *reinterpret_cast<const i32x4*>(brow[q] + 64 * s + 32 * h);
                    const i32x4 b1 = *reinterpret_cast<const i32x4*>(brow[q] + 64 * s + 32 * h + 16);
                    bv[s][q] = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
                }
#pragma unroll
            for (int bm = 0; bm < kBM; ++bm) {
                i32x8 av[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const i32x4 a0 = *reinterpret_cast<const i32x4*>(arow[bm] + 64 * s + 32 * h);
                    const i32x4 a1 = *reinterpret_cast<const i32x4*>(arow[bm] + 64 * s + 32 * h + 16);
                    av[s] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
                }
                float c[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 sx4 =
                        *reinterpret_cast<const f32x4*>(&sx_lds[buf][32 * kBM * wm + 32 * bm + 8 * g + 4 * h]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) c[4 * g + e] = sx4[e] * sw;
                }
#pragma unroll
                for (int bn = 0; bn < 2; ++bn) {
                    f32x16 part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[0], bv[0][bn], zero_f32x16(),
                                                                                   0, 0, 0, 127, 0, 127);
                    part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[1], bv[1][bn], part, 0, 0, 0, 127, 0, 127);
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[bm][bn][i] = fmaf(part[i], c[i], acc[bm][bn][i]);
                }
            }
        }
    };

    // bf16: two steps of loads in flight; FP8 (no registers to spare): one. Step i + 1 goes from
    // registers into the other buffer after step i is multiplied; one barrier per step.
    const int steps = p.k / (kStepBytes / es);
    GemmStage<kBM> ra, rb;
    if constexpr (kFp8) {
        stage_load(ra, 0);
        stage_store(ra, 0);
        __syncthreads();
        for (int i = 0; i < steps; ++i) {
            if (i + 1 < steps) stage_load(ra, i + 1);
            compute(i & 1, i);
            if (i + 1 < steps) stage_store(ra, (i + 1) & 1);
            __syncthreads();
        }
    } else {
        // Unconditional prefetch two steps ahead: loads past the K extent stay inside the rows'
        // buffer range (or read zeros) and are never stored, and with no branch around them the
        // compiler waits for just the older step's loads before each LDS store.
        stage_load(ra, 0);
        stage_store(ra, 0);
        stage_load(ra, 1);
        __syncthreads();
        for (int i = 0; i < steps;) {
            stage_load(rb, i + 2);
            compute(i & 1, i);
            stage_store(ra, (i + 1) & 1);
            __syncthreads();
            if (++i >= steps) break;
            stage_load(ra, i + 2);
            compute(i & 1, i);
            stage_store(rb, (i + 1) & 1);
            __syncthreads();
            ++i;
        }
    }

    // Epilogue: lane column r32 of each block, rows 8 (i / 4) + 4 h + (i % 4).
#pragma unroll
    for (int bm = 0; bm < kBM; ++bm)
#pragma unroll
        for (int bn = 0; bn < 2; ++bn) {
            const int n = n0 + 64 * wn + 32 * bn + r32;
            if (n >= p.n) continue;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + 32 * kBM * wm + 32 * bm + 8 * (i / 4) + 4 * h + (i % 4);
                if (m >= p.m) continue;
                const int64_t off = static_cast<int64_t>(m) * p.ldy + n;
                if (p.y_is_bf16)
                    static_cast<__bf16*>(p.y)[off] = static_cast<__bf16>(acc[bm][bn][i]);
                else
                    static_cast<float*>(p.y)[off] = acc[bm][bn][i];
            }
        }
}

}  // namespace

template <bool kFp8, int kBM>
hipError_t launch_tiles(const GemmParams& p, hipStream_t stream) {
    constexpr int kTileM = 64 * kBM;
    const int64_t tiles = static_cast<int64_t>((p.m + kTileM - 1) / kTileM) * ((p.n + kTileN - 1) / kTileN);
    gemm_bias_kernel<kFp8, kBM><<<dim3(static_cast<unsigned>(tiles)), dim3(kGemmThreads), 0, stream>>>(p);
    return hipGetLastError();
}

hipError_t launch_gemm_bias(const GemmParams& p, bool fp8, hipStream_t stream) {
    return fp8 ? launch_tiles<true, kGemmBM>(p, stream) : launch_tiles<false, kGemmBM>(p, stream);
}

}  // namespace sinkattn
