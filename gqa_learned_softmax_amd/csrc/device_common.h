// Device-side helpers shared by the sink-attention kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

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

// Lane-crossing max/sum over the lanes l, l^16, l^32, l^48 (the four k-slot groups of one MFMA
// column).
__device__ __forceinline__ float max_over_groups(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

__device__ __forceinline__ float sum_over_groups(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    bf16x8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
    return z;
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

// Compiler-level ordering of LDS accesses made by one wave. The hardware executes one wave's LDS
// instructions in order, so a wave-private LDS region needs no s_barrier.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

}  // namespace sinkattn
