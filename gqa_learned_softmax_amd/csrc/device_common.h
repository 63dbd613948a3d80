// Device-side helpers shared by the sink-attention kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Debug builds only; the shipped library defines none of these.
//  SINKATTN_POISON_LDS: every LDS staging buffer is filled with NaN before each refill (and once at
//    the start), so a read that races its refill, or reads a part no refill writes, puts NaN into
//    the output instead of going unnoticed with stale values.
//  SINKATTN_MUTATE_SINK_EVERY_CHUNK: every KV chunk (decode) and split (prefill) starts from the
//    sink, not only the first one -- a deliberate mistake the parity tests must catch.
//  SINKATTN_MUTATE_D0_ZERO: rows start at m = sink with d = 0, so the sink sets the starting
//    reference but adds nothing to the denominator -- likewise a deliberate mistake.
#ifdef SINKATTN_POISON_LDS
constexpr bool kPoisonLds = true;
#else
constexpr bool kPoisonLds = false;
#endif
#ifdef SINKATTN_MUTATE_SINK_EVERY_CHUNK
constexpr bool kMutateSinkEveryChunk = true;
#else
constexpr bool kMutateSinkEveryChunk = false;
#endif
#ifdef SINKATTN_MUTATE_D0_ZERO
constexpr bool kMutateD0Zero = true;
#else
constexpr bool kMutateD0Zero = false;
#endif

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// A (16x32) times B (32x16), bf16 inputs, fp32 16x16 accumulator: v_mfma_f32_16x16x32_bf16.
// Operand layout (lane l, 64 lanes): A holds row (l % 16) and 8 consecutive k-slots of group
// (l / 16); B holds column (l % 16) and the same 8 k-slots; the result holds rows
// 4 * (l / 16) + 0..3 of column (l % 16). Any permutation of the k index applied identically to A
// and B leaves the product unchanged, which the kernels use to match register layouts.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A (16x16) times B (16x16), bf16 inputs, fp32 16x16 accumulator: v_mfma_f32_16x16x16_bf16.
// Lane l: A holds row (l % 16) and the 4 k-slots 4 * (l / 16) + 0..3; B holds column (l % 16) and
// the same k-slots; the result holds rows 4 * (l / 16) + 0..3 of column (l % 16), which is the
// B-operand layout again, so a 16x16x32 accumulator's 4 values per lane are ready P^T operands.
__device__ __forceinline__ f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// A (32x16) times B (16x32), bf16 inputs, fp32 32x32 accumulator: v_mfma_f32_32x32x16_bf16.
// Lane l: A holds row (l % 32) and 8 k-slots of group (l / 32); B holds column (l % 32) and the
// same k-slots; result register r holds row 8 * (r / 4) + 4 * (l / 32) + (r % 4) of column
// (l % 32). On gfx950 this shape sustains close to twice the throughput of the 16x16x32 one.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero_f32x16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// gfx950 LDS transpose read (ds_read_b64_tr_b16). Within each group of 16 lanes, result lane i,
// element e is element (i % 4) of the 8-byte row addressed by lane 4 * e + i / 4 of the same
// group. So if lane 4e + j of a group points at row r_e, columns c0 + 4j .. c0 + 4j + 3 of a
// row-major bf16 tile, lane i receives column c0 + i of rows r_0 .. r_3: a 4 x 16 block comes
// back transposed, ready as 4 k-slots of an MFMA operand.
__device__ __forceinline__ bf16x4 lds_read_tr4(const __bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4*)(const_cast<__bf16*>(p)));
}

// Values of lanes l ^ 32 and l ^ 16 through the gfx950 lane-swap instructions (VALU only, no LDS
// round trip). With both operands equal, v_permlane32_swap returns the low half duplicated and the
// high half duplicated, so every lane sees its own value and its partner's.
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max/sum over the lanes l, l^16, l^32, l^48 (the four k-slot groups of one 16x16 MFMA column).
__device__ __forceinline__ float max_over_groups(float x) { return max_xor32(max_xor16(x)); }

__device__ __forceinline__ float sum_over_groups(float x) { return sum_xor32(sum_xor16(x)); }

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    bf16x8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
    return z;
}

// Eight bf16 quiet NaNs (bit pattern 0x7FC0), the poison of SINKATTN_POISON_LDS builds.
__device__ __forceinline__ bf16x8 nan_bf16x8() {
    typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
    const u16x8 bits = {0x7FC0, 0x7FC0, 0x7FC0, 0x7FC0, 0x7FC0, 0x7FC0, 0x7FC0, 0x7FC0};
    return __builtin_bit_cast(bf16x8, bits);
}

__device__ __forceinline__ f32x4 zero_f32x4() { return f32x4{0.0f, 0.0f, 0.0f, 0.0f}; }

// Raw buffer resource over [base, base + num_bytes). A buffer load whose offset lies past
// num_bytes returns zeros and makes no memory access, so tails and prefetches past the end need
// neither a branch nor an exec-mask change (branch-free loads also let the compiler keep exact
// s_waitcnt vmcnt counts across a software-pipelined loop). Dword 3 = 0x00020000 selects the
// 32-bit data format that gfx9-family raw buffer accesses require.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_buffer(const void* base, uint32_t num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(num_bytes), 0x00020000);
}

__device__ __forceinline__ bf16x8 buffer_load_x8(__amdgpu_buffer_rsrc_t rsrc, uint32_t byte_offset) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rsrc, byte_offset, 0, 0));
}

// The same load with the non-temporal hint (bit 1 of the cache-policy operand, `nt` on gfx950), for
// data a kernel streams through once: the lines are not kept in the caches, which on MI355X made
// the split-KV decode kernels' K/V stream 7-11% faster (8 x 8192 keys: 27.9 -> 25.0 us).
__device__ __forceinline__ bf16x8 buffer_load_x8_stream(__amdgpu_buffer_rsrc_t rsrc, uint32_t byte_offset) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rsrc, byte_offset, 0, 2));
}

// acc + p[0] + p[1] in fp32 with one v_dot2c_f32_bf16 against (1, 1).
__device__ __forceinline__ float sum_bf16x2(bf16x2 p, float acc) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(p, ones, acc, false);
}

// Scheduling hint for the current scheduling region: alternate one MFMA with kValu VALU
// instructions, kMfma times, so the matrix core and the vector ALU of one wave stay busy together.
template <int kMfma, int kValu>
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);  // VALU
    }
}

// Compiler-level ordering of LDS accesses made by one wave. The hardware executes one wave's LDS
// instructions in order, so a wave-private LDS region needs no s_barrier.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

}  // namespace sinkattn
