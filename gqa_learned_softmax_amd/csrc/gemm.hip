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

constexpr int kStepBytes = 128;    // bytes of each row staged per K step
constexpr int kRowPitch = 144;     // LDS row pitch in bytes
constexpr int kGroupRows = 8;      // tile-rows per group in the tile order

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Work-group layout: kWM x kWN waves, each owning kBM x kBN blocks of 32 x 32, so the tile is
// (32 kBM kWM) x (32 kBN kWN). A step stages 8 sixteen-byte pieces per tile row.
template <int kBM, int kBN, int kWM, int kWN>
struct GemmShape {
    static constexpr int kThreads = 64 * kWM * kWN;
    static constexpr int kTileM = 32 * kBM * kWM;
    static constexpr int kTileN = 32 * kBN * kWN;
    static constexpr int kPiecesA = kTileM * 8 / kThreads;
    static constexpr int kPiecesB = kTileN * 8 / kThreads;
    static_assert(kTileM * 8 % kThreads == 0 && kTileN * 8 % kThreads == 0, "whole pieces per thread");
    static_assert(kThreads >= kTileM, "one row scale per thread");
    static_assert(kTileN % 128 == 0 && 128 % (32 * kBN) == 0, "a wave's columns share one weight scale");
};

template <class S>
struct GemmStage {
    i32x4 a[S::kPiecesA];
    i32x4 b[S::kPiecesB];
    float sx;  // FP8: the scale of tile row tid (threads below the tile's row count)
};

template <bool kFp8, int kBM, int kBN, int kWM, int kWN>
__global__ __launch_bounds__(64 * kWM * kWN, kWM * kWN == 4 ? 2 : 1) void gemm_bias_kernel(GemmParams p) {
    using S = GemmShape<kBM, kBN, kWM, kWN>;
    constexpr int kThreads = S::kThreads, kTileM = S::kTileM, kTileN = S::kTileN;
    __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][kTileM][kRowPitch];
    __shared__ __attribute__((aligned(16))) uint8_t b_lds[2][kTileN][kRowPitch];
    __shared__ __attribute__((aligned(16))) float sx_lds[2][kTileM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWN, wn = wave % kWN;
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
    f32x16 acc[kBM][kBN];
#pragma unroll
    for (int bn = 0; bn < kBN; ++bn) {
        const int n = n0 + 32 * kBN * wn + 32 * bn + r32;
        const float b = p.bias != nullptr && n < p.n ? p.bias[n] : 0.0f;
#pragma unroll
        for (int bm = 0; bm < kBM; ++bm)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[bm][bn][i] = b;
    }

    // Thread piece j: row (tid + T j) / 8, 16-byte segment (tid + T j) % 8 of the step's bytes.
    auto stage_load = [&](GemmStage<S>& st, int step) {
        const uint32_t kb = static_cast<uint32_t>(step) * kStepBytes;
#pragma unroll
        for (int j = 0; j < S::kPiecesA; ++j) {
            const int piece = tid + kThreads * j;
            const uint32_t row = piece >> 3, seg = piece & 7;
            st.a[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, row * lda + kb + 16 * seg, 0, 0));
        }
#pragma unroll
        for (int j = 0; j < S::kPiecesB; ++j) {
            const int piece = tid + kThreads * j;
            const uint32_t row = piece >> 3, seg = piece & 7;
            st.b[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(brs, row * ldb + kb + 16 * seg, 0, 0));
        }
        if constexpr (kFp8) {
            const int row = m0 + tid;
            st.sx = tid < kTileM && row < p.m ? p.scale_x[row * p.sx_stride_m + step * p.sx_stride_kb] : 0.0f;
        }
    };
    auto stage_store = [&](const GemmStage<S>& st, int buf) {
#pragma unroll
        for (int j = 0; j < S::kPiecesA; ++j) {
            const int piece = tid + kThreads * j;
            *reinterpret_cast<i32x4*>(&a_lds[buf][piece >> 3][16 * (piece & 7)]) = st.a[j];
        }
#pragma unroll
        for (int j = 0; j < S::kPiecesB; ++j) {
            const int piece = tid + kThreads * j;
            *reinterpret_cast<i32x4*>(&b_lds[buf][piece >> 3][16 * (piece & 7)]) = st.b[j];
        }
        if constexpr (kFp8)
            if (tid < kTileM) sx_lds[buf][tid] = st.sx;
    };
    auto compute = [&](int buf, int step) {
        const uint8_t* arow[kBM];
        const uint8_t* brow[kBN];
#pragma unroll
        for (int q = 0; q < kBM; ++q) arow[q] = &a_lds[buf][32 * kBM * wm + 32 * q + r32][0];
#pragma unroll
        for (int q = 0; q < kBN; ++q) brow[q] = &b_lds[buf][32 * kBN * wn + 32 * q + r32][0];
        if constexpr (!kFp8) {
            // Four k slices of 16 bf16; lane half h takes k 8h .. 8h + 7 of each slice.
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf16x8 av[kBM], bv[kBN];
#pragma unroll
                for (int q = 0; q < kBM; ++q) av[q] = *reinterpret_cast<const bf16x8*>(arow[q] + 32 * kk + 16 * h);
#pragma unroll
                for (int q = 0; q < kBN; ++q) bv[q] = *reinterpret_cast<const bf16x8*>(brow[q] + 32 * kk + 16 * h);
#pragma unroll
                for (int bm = 0; bm < kBM; ++bm)
#pragma unroll
                    for (int bn = 0; bn < kBN; ++bn) acc[bm][bn] = mfma32x32x16(av[bm], bv[bn], acc[bm][bn]);
            }
        } else {
            // Two k slices of 64 FP8; lane half h takes bytes 32h .. 32h + 31 of each slice (the
            // same bytes for A and B, so the product pairs equal k whatever order the unit uses).
            // Each block's two products go into a temporary that is promoted at once:
            // acc += part * scale_x[row] * scale_w (the wave's columns share one weight scale).
            const int nb = (n0 + 32 * kBN * wn) / 128;
            const float sw = p.scale_w[static_cast<int64_t>(nb) * p.sw_stride_nb + step * p.sw_stride_kb];
            i32x8 bv[2][kBN];
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int q = 0; q < kBN; ++q) {
                    const i32x4 b0 = *reinterpret_cast<const i32x4*>(brow[q] + 64 * sl + 32 * h);
                    const i32x4 b1 = *reinterpret_cast<const i32x4*>(brow[q] + 64 * sl + 32 * h + 16);
                    bv[sl][q] = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
                }
#pragma unroll
            for (int bm = 0; bm < kBM; ++bm) {
                i32x8 av[2];
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) {
                    const i32x4 a0 = *reinterpret_cast<const i32x4*>(arow[bm] + 64 * sl + 32 * h);
                    const i32x4 a1 = *reinterpret_cast<const i32x4*>(arow[bm] + 64 * sl + 32 * h + 16);
                    av[sl] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
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
                for (int bn = 0; bn < kBN; ++bn) {
                    f32x16 part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[0], bv[0][bn], zero_f32x16(),
                                                                                   0, 0, 0, 127, 0, 127);
                    part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[1], bv[1][bn], part, 0, 0, 0, 127, 0, 127);
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[bm][bn][i] = fmaf(part[i], c[i], acc[bm][bn][i]);
                }
            }
        }
    };

    // bf16 with four waves: two steps of loads in flight; FP8 and the eight-wave tiles (no registers
    // to spare): one. Step i + 1 goes from registers into the other buffer after step i is
    // multiplied; one barrier per step.
    const int steps = p.k / (kStepBytes / es);
    GemmStage<S> ra, rb;
    if constexpr (kFp8 || kWM * kWN > 4) {
        stage_load(ra, 0);
        stage_store(ra, 0);
        __syncthreads();
        for (int i = 0; i < steps; ++i) {
            if (i + 1 < steps) stage_load(ra, i + 1);
            // bf16: a wave issuing its MFMAs goes ahead of its SIMD partner's LDS stores (measured
            // 2-3% faster at 4096^3 and 8192 x 8192 x 4096; FP8 measured slower with it).
            if constexpr (!kFp8) __builtin_amdgcn_s_setprio(1);
            compute(i & 1, i);
            if constexpr (!kFp8) __builtin_amdgcn_s_setprio(0);
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
        for (int bn = 0; bn < kBN; ++bn) {
            const int n = n0 + 32 * kBN * wn + 32 * bn + r32;
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

template <bool kFp8, int kBM, int kBN, int kWM, int kWN>
hipError_t launch_shape(const GemmParams& p, hipStream_t stream) {
    using S = GemmShape<kBM, kBN, kWM, kWN>;
    const int64_t tiles = static_cast<int64_t>((p.m + S::kTileM - 1) / S::kTileM) * ((p.n + S::kTileN - 1) / S::kTileN);
    gemm_bias_kernel<kFp8, kBM, kBN, kWM, kWN>
        <<<dim3(static_cast<unsigned>(tiles)), dim3(S::kThreads), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace

// FP8: 128 x 128 tiles, four waves of 2 x 2 blocks (two work-groups per CU). bf16: 256 x 256 tiles,
// eight waves of 4 x 2 blocks, where the problem has rows and columns for them (fewer operand
// reads and LDS writes per flop); 128 x 128 otherwise.
hipError_t launch_gemm_bias(const GemmParams& p, bool fp8, hipStream_t stream) {
    if (fp8) return launch_shape<true, 2, 2, 2, 2>(p, stream);
    if (p.m >= 256 && p.n >= 256) return launch_shape<false, 4, 2, 2, 4>(p, stream);
    return launch_shape<false, 2, 2, 2, 2>(p, stream);
}

}  // namespace sinkattn
