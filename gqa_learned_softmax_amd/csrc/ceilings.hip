// Measured ceilings of the MI355X that runs the library: the rate at which a plain kernel streams
// bytes out of HBM, the rate at which the matrix cores retire bf16 MFMAs at the clock the chip
// holds under that load, and what the instructions of the prefill's inner loop cost a SIMD. They
// are the denominators the benchmark reports beside the published peaks (8 TB/s HBM, 2.5 PFLOP/s
// dense bf16). Measurement only: nothing in libsinkattn calls them, and they are built into a
// library of their own (libsinkattn_ceilings.so).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sinkattn_ceilings.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Every byte of buf read once with non-temporal 16-byte loads (the hint the decode kernels use for
// their K/V stream). Grid-stride over 16-byte pieces with four loads in flight per thread; each
// iteration of the grid reads one contiguous span. The XOR of everything read goes to out only if
// it equals a value it cannot equal by construction of the caller's fill, so the loads stay live
// without a store per thread.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ buf, uint64_t pieces,
                                                          uint32_t* out) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + 3 * stride < pieces; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(buf + i);
        const u32x4 b = __builtin_nontemporal_load(buf + i + stride);
        const u32x4 c = __builtin_nontemporal_load(buf + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(buf + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < pieces; i += stride) acc ^= __builtin_nontemporal_load(buf + i);
    const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == 0x9E3779B9u) out[0] = x;
}

// The split-KV decode's read pattern with nothing else: two row-major tensors (a token-major K and V
// cache) of seqs x chunks x rows_per_chunk rows, every 256-byte slice of every row read once with
// non-temporal 16-byte loads. Work-group w takes slice w % S (S = row_pieces / 16) of the rows of
// chunk g / seqs of sequence g % seqs, g = w / S (the decode's order: KV-head pair fastest, then the
// sequence, then the chunk); its 512 threads read pieces j = tid + 512 u of the chunk's slice (16
// per row), two of K and two of V in flight per thread.
__global__ __launch_bounds__(512) void stream_read_slices_kernel(const u32x4* __restrict__ k,
                                                                 const u32x4* __restrict__ v, uint32_t row_pieces,
                                                                 uint32_t seqs, uint32_t chunks,
                                                                 uint32_t rows_per_chunk, uint32_t* out) {
    const uint32_t slices = row_pieces / 16;
    const uint32_t w = blockIdx.x;
    const uint32_t slice = w % slices;
    const uint32_t g = w / slices;
    const uint64_t row0 = (static_cast<uint64_t>(g % seqs) * chunks + g / seqs) * rows_per_chunk;
    const uint32_t pieces = rows_per_chunk * 16;
    auto at = [&](uint32_t j) { return (row0 + j / 16) * row_pieces + slice * 16 + j % 16; };
    u32x4 acc = {0u, 0u, 0u, 0u};
    uint32_t j = threadIdx.x;
    for (; j + 512 < pieces; j += 1024) {
        const u32x4 a = __builtin_nontemporal_load(k + at(j));
        const u32x4 b = __builtin_nontemporal_load(k + at(j + 512));
        const u32x4 c = __builtin_nontemporal_load(v + at(j));
        const u32x4 d = __builtin_nontemporal_load(v + at(j + 512));
        acc ^= a ^ b ^ c ^ d;
    }
    for (; j < pieces; j += 512) acc ^= __builtin_nontemporal_load(k + at(j)) ^ __builtin_nontemporal_load(v + at(j));
    const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == 0x9E3779B9u) out[0] = x;
}

// Four independent accumulation chains of v_mfma_f32_32x32x16_bf16 per wave, so consecutive MFMAs
// never wait on each other's results; operands come from the thread index so nothing folds away.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* out) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = static_cast<__bf16>(static_cast<float>((threadIdx.x + e) & 7) * 0.125f);
        b[e] = static_cast<__bf16>(static_cast<float>((threadIdx.x * 3 + e) & 7) * 0.0625f);
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    if (s == -1.0f) out[0] = s;  // never true for these operands (every product is >= 0)
}

// The same MFMA loop on operands that look like real data: four A and four B operands per lane of
// uniform random bf16 values in [-2, 2) (full mantissas, from a per-thread xorshift), cycled so that
// consecutive MFMAs never share an operand. The chip's clock under MFMA work depends on how many
// operand bits switch, so this rate is the one a kernel multiplying random bf16 data can approach.
// Eight MFMAs per iteration (four chains of two).
__global__ __launch_bounds__(256) void mfma_random_kernel(int iters, float* out) {
    uint32_t h = (blockIdx.x * 256u + threadIdx.x) * 0x9E3779B9u + 0x7F4A7C15u;
    auto next = [&]() {
        h ^= h << 13;
        h ^= h >> 17;
        h ^= h << 5;
        return static_cast<__bf16>(static_cast<float>(static_cast<int>(h & 0xFFFFu) - 32768) * (1.0f / 16384.0f));
    };
    bf16x8 a0, a1, a2, a3, b0, b1, b2, b3;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a0[e] = next(); a1[e] = next(); a2[e] = next(); a3[e] = next();
        b0[e] = next(); b1[e] = next(); b2[e] = next(); b3[e] = next();
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b2, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3, b3, c3, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b2, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b3, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3, b0, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, c3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    if (s == 1234567.0f) out[0] = s;  // keeps the products live; the value is never this
}

// Issue-cost loops: each wave repeats one fixed group of instructions on eight rotating fp32
// registers and independent accumulators, so (kinds 0-6) nothing waits on a recent result and the
// time per group is what the instructions themselves cost the SIMD; kind 7 chains each multiply
// into an exponential and pairs of those into a pack, as the prefill does per score. Wave 0 of each work-group records the shader-clock
// cycles (s_memtime) and 100 MHz ticks (s_memrealtime) its loop took, from which the caller gets
// the clock. The vector instructions are written as asm so the compiler neither folds nor reorders
// them; they only read and write registers.
#define SA_EXP(r) asm volatile("v_exp_f32 %0, %0" : "+v"(r))
#define SA_MUL(r) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(r) : "v"(k))
#define SA_FMA(r) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(r) : "v"(k), "v"(k2))
#define SA_CVT(d, a, b) asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b))
#define SA_MFMA32(c) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0)
#define SA_MFMA16(c) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0)
#define SA_EXP8 SA_EXP(r0); SA_EXP(r1); SA_EXP(r2); SA_EXP(r3); SA_EXP(r4); SA_EXP(r5); SA_EXP(r6); SA_EXP(r7)
#define SA_MUL8 SA_MUL(r0); SA_MUL(r1); SA_MUL(r2); SA_MUL(r3); SA_MUL(r4); SA_MUL(r5); SA_MUL(r6); SA_MUL(r7)
#define SA_FMA8 SA_FMA(r0); SA_FMA(r1); SA_FMA(r2); SA_FMA(r3); SA_FMA(r4); SA_FMA(r5); SA_FMA(r6); SA_FMA(r7)
#define SA_CVT8 SA_CVT(d0, r0, r1); SA_CVT(d1, r2, r3); SA_CVT(d2, r4, r5); SA_CVT(d3, r6, r7); \
    SA_CVT(d0, r1, r0); SA_CVT(d1, r3, r2); SA_CVT(d2, r5, r4); SA_CVT(d3, r7, r6)

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int kKind>
__global__ __launch_bounds__(256) void issue_kernel(int iters, unsigned long long* clk, float* out) {
    const float k = 0.9990234375f, k2 = 0.5f;
    float r0 = threadIdx.x * 1e-3f, r1 = r0 + 1.0f, r2 = r0 + 2.0f, r3 = r0 + 3.0f, r4 = r0 - 1.0f,
          r5 = r0 - 2.0f, r6 = r0 - 3.0f, r7 = r0 - 4.0f;
    int d0 = 0, d1 = 0, d2 = 0, d3 = 0;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = static_cast<__bf16>(static_cast<float>((threadIdx.x + e) & 7) * 0.125f);
        b[e] = static_cast<__bf16>(static_cast<float>((threadIdx.x * 3 + e) & 7) * 0.0625f);
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    f32x4 s0 = {}, s1 = {};
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long q0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        if constexpr (kKind == 0) {  // 16 v_exp_f32
            SA_EXP8; SA_EXP8;
        } else if constexpr (kKind == 1) {  // 16 v_mul_f32
            SA_MUL8; SA_MUL8;
        } else if constexpr (kKind == 2) {  // 16 v_cvt_pk_bf16_f32
            SA_CVT8; SA_CVT8;
        } else if constexpr (kKind == 3) {  // 16 v_fma_f32
            SA_FMA8; SA_FMA8;
        } else if constexpr (kKind == 4) {  // 4 v_mfma_f32_32x32x16_bf16
            SA_MFMA32(c0); SA_MFMA32(c1); SA_MFMA32(c2); SA_MFMA32(c3);
        } else if constexpr (kKind == 5) {  // 4 v_mfma_f32_16x16x32_bf16
            SA_MFMA16(s0); SA_MFMA16(s1); SA_MFMA16(s0); SA_MFMA16(s1);
        } else if constexpr (kKind == 6) {  // 4 32x32x16 MFMAs, each followed by 4 exponentials
            SA_MFMA32(c0); SA_EXP(r0); SA_EXP(r1); SA_EXP(r2); SA_EXP(r3);
            SA_MFMA32(c1); SA_EXP(r4); SA_EXP(r5); SA_EXP(r6); SA_EXP(r7);
            SA_MFMA32(c2); SA_EXP(r0); SA_EXP(r1); SA_EXP(r2); SA_EXP(r3);
            SA_MFMA32(c3); SA_EXP(r4); SA_EXP(r5); SA_EXP(r6); SA_EXP(r7);
        } else {  // a quarter of the prefill's per-tile mix: 8 + 2 MFMAs, 16 mul -> exp, 8 cvt
            SA_MFMA32(c0); SA_MUL(r0); SA_EXP(r0); SA_MUL(r1); SA_EXP(r1);
            SA_MFMA32(c1); SA_CVT(d0, r0, r1); SA_MUL(r2); SA_EXP(r2);
            SA_MFMA32(c2); SA_MUL(r3); SA_EXP(r3); SA_CVT(d1, r2, r3);
            SA_MFMA32(c3); SA_MUL(r4); SA_EXP(r4); SA_MUL(r5); SA_EXP(r5);
            SA_MFMA16(s0); SA_CVT(d2, r4, r5); SA_MUL(r6); SA_EXP(r6);
            SA_MFMA32(c0); SA_MUL(r7); SA_EXP(r7); SA_CVT(d3, r6, r7);
            SA_MFMA32(c1); SA_MUL(r0); SA_EXP(r0); SA_MUL(r1); SA_EXP(r1);
            SA_MFMA32(c2); SA_CVT(d0, r0, r1); SA_MUL(r2); SA_EXP(r2);
            SA_MFMA32(c3); SA_MUL(r3); SA_EXP(r3); SA_CVT(d1, r2, r3);
            SA_MFMA16(s1); SA_MUL(r4); SA_EXP(r4); SA_MUL(r5); SA_EXP(r5); SA_CVT(d2, r4, r5);
            SA_MUL(r6); SA_EXP(r6); SA_MUL(r7); SA_EXP(r7); SA_CVT(d3, r6, r7);
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long q1 = __builtin_amdgcn_s_memrealtime();
    float sum = r0 + r1 + r2 + r3 + r4 + r5 + r6 + r7 + static_cast<float>(d0 ^ d1 ^ d2 ^ d3) + s0[0] + s1[1];
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += c0[r] + c1[r] + c2[r] + c3[r];
    if (sum == -12345.0f) out[0] = sum;  // keeps the results live
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = t1 - t0;
        clk[2 * blockIdx.x + 1] = q1 - q0;
    }
}

#undef SA_EXP8
#undef SA_MUL8
#undef SA_FMA8
#undef SA_CVT8

}  // namespace

extern "C" {

int sinkattn_ceiling_stream_read(const void* buf, uint64_t bytes, int blocks, void* out4, void* stream) {
    if (buf == nullptr || out4 == nullptr || blocks <= 0 || bytes % 16 != 0 ||
        reinterpret_cast<uintptr_t>(buf) % 16 != 0)
        return 1;
    stream_read_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4*>(buf), bytes / 16, static_cast<uint32_t*>(out4));
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int sinkattn_ceiling_stream_read_slices(const void* k, const void* v, int seqs, int chunks, int rows_per_chunk,
                                        int row_bytes, void* out4, void* stream) {
    if (k == nullptr || v == nullptr || out4 == nullptr || seqs <= 0 || chunks <= 0 || rows_per_chunk <= 0 ||
        row_bytes <= 0 || row_bytes % 256 != 0 || reinterpret_cast<uintptr_t>(k) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(v) % 16 != 0)
        return 1;
    const int64_t groups = static_cast<int64_t>(seqs) * chunks * (row_bytes / 256);
    const int64_t rows = static_cast<int64_t>(seqs) * chunks * rows_per_chunk;
    if (groups > 0x7FFFFFFF || static_cast<int64_t>(rows_per_chunk) * 16 > 0x7FFFFFFF || rows > (int64_t(1) << 40))
        return 1;
    stream_read_slices_kernel<<<dim3(static_cast<unsigned>(groups)), dim3(512), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), static_cast<uint32_t>(row_bytes / 16),
        static_cast<uint32_t>(seqs), static_cast<uint32_t>(chunks), static_cast<uint32_t>(rows_per_chunk),
        static_cast<uint32_t*>(out4));
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int sinkattn_ceiling_mfma_bf16(int blocks, int iters, void* out4, void* stream) {
    if (out4 == nullptr || blocks <= 0 || iters <= 0) return 1;
    mfma_loop_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
        iters, static_cast<float*>(out4));
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int sinkattn_ceiling_mfma_bf16_random(int blocks, int iters, void* out4, void* stream) {
    if (out4 == nullptr || blocks <= 0 || iters <= 0) return 1;
    mfma_random_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
        iters, static_cast<float*>(out4));
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

double sinkattn_ceiling_mfma_bf16_random_flop(int blocks, int iters) {
    // 4 waves per block, 8 MFMAs per iteration, 32 x 32 x 16 x 2 flop each.
    return static_cast<double>(blocks) * 4.0 * iters * 8.0 * 32.0 * 32.0 * 16.0 * 2.0;
}

double sinkattn_ceiling_mfma_bf16_flop(int blocks, int iters) {
    // 4 waves per block, 4 MFMAs per iteration, 32 x 32 x 16 x 2 flop each.
    return static_cast<double>(blocks) * 4.0 * iters * 4.0 * 32.0 * 32.0 * 16.0 * 2.0;
}

int sinkattn_ceiling_issue(int kind, int blocks, int iters, void* clk, void* out4, void* stream) {
    if (clk == nullptr || out4 == nullptr || blocks <= 0 || iters <= 0 || kind < 0 || kind > 7) return 1;
    const dim3 grid(static_cast<unsigned>(blocks)), block(256);
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto* c = static_cast<unsigned long long*>(clk);
    auto* o = static_cast<float*>(out4);
    switch (kind) {
        case 0: issue_kernel<0><<<grid, block, 0, st>>>(iters, c, o); break;
        case 1: issue_kernel<1><<<grid, block, 0, st>>>(iters, c, o); break;
        case 2: issue_kernel<2><<<grid, block, 0, st>>>(iters, c, o); break;
        case 3: issue_kernel<3><<<grid, block, 0, st>>>(iters, c, o); break;
        case 4: issue_kernel<4><<<grid, block, 0, st>>>(iters, c, o); break;
        case 5: issue_kernel<5><<<grid, block, 0, st>>>(iters, c, o); break;
        case 6: issue_kernel<6><<<grid, block, 0, st>>>(iters, c, o); break;
        default: issue_kernel<7><<<grid, block, 0, st>>>(iters, c, o); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
