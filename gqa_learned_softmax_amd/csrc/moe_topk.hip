// MoE routing weights: top-K experts per token, softmax over the K chosen logits (gfx950).
//
// Source: "GPT-OSS on Day 0" (Perplexity): the model outline ("GPT-OSS on Hopper") lists a softmax
// after the top-K choice for the expert weights, and section "Kernels for GPT-OSS" says the routing
// scores take the softmax over the top-K chosen experts only (where DeepSeek-style models take it
// over all experts) and that the expert weights must be computed in bfloat16 for accuracy. Here the
// softmax runs in fp32 on the chosen logits and the weights are stored rounded to bf16 (or as fp32);
// the all-experts normalisation is kept as a mode for contrast.
//
// Streaming kernel: one 16-lane group per token row (four rows per wave; a group is one DPP row).
// Lane j of a group holds logits [j V, j V + V), V = E / 16 rounded up to a power of two (16-byte
// loads when the row fills the group exactly and rows are 16-byte aligned; element loads
// otherwise). K rounds each find the group's largest remaining logit (ties: lower expert index)
// with four row-local DPP steps, and lane r of the group keeps round r's choice. bf16 logits go
// through 32-bit keys that pack (value, expert) in selection order: each lane sorts its V keys once
// (a compare-exchange network), and a round is the group max of the list heads plus a one-place
// shift in the winning lane. fp32 logits compare (value, index) pairs element by element. Lanes
// r < K then hold the chosen (logit, id) in order and write their weight and id.

#include "device_common.h"
#include "launch_ops.h"

namespace sinkattn {
namespace {

constexpr int kMoeThreads = 256;
constexpr int kGroupLanes = 16;

// (value, index) order of the selection: larger value first, then lower index. Bitwise operators,
// not short-circuit ones, so the compiler emits selects rather than exec-mask branches.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return (v > bv) | ((v == bv) & (i < bi));
}

// A 16-lane group is one DPP row. Butterfly over it with row-local DPP moves (no LDS crossbar):
// swap neighbours, swap pairs (quad permutes), mirror within each half row, mirror the row. After
// the four steps every lane holds the reduction of all 16.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror

template <int kCtrl>
__device__ __forceinline__ int row_move(int x) {
    return __builtin_amdgcn_update_dpp(0, x, kCtrl, 0xF, 0xF, false);
}

template <int kCtrl>
__device__ __forceinline__ void keep_better(float& v, int& i) {
    const float ov = __int_as_float(row_move<kCtrl>(__float_as_int(v)));
    const int oi = row_move<kCtrl>(i);
    if (better(ov, oi, v, i)) {
        v = ov;
        i = oi;
    }
}

__device__ __forceinline__ void group_best(float& v, int& i) {
    keep_better<kDppXor1>(v, i);
    keep_better<kDppXor2>(v, i);
    keep_better<kDppHalfMirror>(v, i);
    keep_better<kDppMirror>(v, i);
}

template <int kCtrl>
__device__ __forceinline__ float add_moved(float x) {
    return x + __int_as_float(row_move<kCtrl>(__float_as_int(x)));
}

__device__ __forceinline__ float group_sum(float x) {
    x = add_moved<kDppXor1>(x);
    x = add_moved<kDppXor2>(x);
    x = add_moved<kDppHalfMirror>(x);
    return add_moved<kDppMirror>(x);
}

template <int kCtrl>
__device__ __forceinline__ uint32_t max_moved(uint32_t x) {
    const uint32_t o = static_cast<uint32_t>(row_move<kCtrl>(static_cast<int>(x)));
    return x > o ? x : o;
}

__device__ __forceinline__ uint32_t group_max(uint32_t x) {
    x = max_moved<kDppXor1>(x);
    x = max_moved<kDppXor2>(x);
    x = max_moved<kDppHalfMirror>(x);
    return max_moved<kDppMirror>(x);
}

// bf16 logits: (value, expert) packed into one 32-bit key whose unsigned order is the selection
// order. The logit's fp32 bits f (bf16 bits << 16: the low half is zero) go from sign-magnitude to
// two's complement, s = f >= 0 ? f : INT_MIN - f, which orders them as floats order them, with -0
// and +0 both 0; adding 2^31 makes the order unsigned, and the zero low half takes 0xFFFF - expert,
// so among equal values the lower expert has the larger key. Keys are unique, and 0 is below every
// key of a real logit (NaN excluded), so it marks padding.
__device__ __forceinline__ uint32_t bf16_key(uint32_t f, int expert) {
    const int32_t si = static_cast<int32_t>(f);
    const int32_t neg = si >> 31;                       // all ones for negative logits
    const int32_t twos = (si ^ (neg & 0x7FFFFFFF)) - neg;  // INT_MIN - f for negative f
    return static_cast<uint32_t>(twos) + 0x80000000u + (0xFFFFu - static_cast<uint32_t>(expert));
}

__device__ __forceinline__ float key_value(uint32_t key) {
    const int32_t twos = static_cast<int32_t>((key & 0xFFFF0000u) - 0x80000000u);
    const int32_t neg = twos >> 31;
    return __int_as_float((twos + neg) ^ (neg & 0x7FFFFFFF));
}

__device__ __forceinline__ int key_expert(uint32_t key) { return static_cast<int>(0xFFFFu - (key & 0xFFFFu)); }

// Sorts V keys into descending order in registers: Batcher's odd-even merge network (19
// compare-exchanges for V = 8), fully unrolled so every index is a constant.
template <int V>
__device__ __forceinline__ void sort_desc(uint32_t (&k)[V]) {
#pragma unroll
    for (int p = 1; p < V; p <<= 1)
#pragma unroll
        for (int q = p; q >= 1; q >>= 1)
#pragma unroll
            for (int j = q % p; j + q < V; j += 2 * q)
#pragma unroll
                for (int i = 0; i < q; ++i)
                    if ((i + j) / (2 * p) == (i + j + q) / (2 * p)) {
                        const uint32_t a = k[i + j], b = k[i + j + q];
                        k[i + j] = a > b ? a : b;
                        k[i + j + q] = a > b ? b : a;
                    }
}

// bf16 logits: lane j's keys of logits [j V, j V + V) (padding: key 0).
template <int V>
__device__ __forceinline__ void load_keys(const MoeTopkParams& p, int64_t row, int j, uint32_t (&key)[V]) {
    const __bf16* row_start = static_cast<const __bf16*>(p.logits) + row * p.logits_stride;
    if (p.vector_rows && p.experts == kGroupLanes * V && V >= 8) {
#pragma unroll
        for (int h = 0; h < V / 8; ++h) {
            const i32x4 w4 = *reinterpret_cast<const i32x4*>(row_start + j * V + 8 * h);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t w = static_cast<uint32_t>(w4[e / 2]);
                const uint32_t f = e % 2 ? w & 0xFFFF0000u : w << 16;
                key[8 * h + e] = bf16_key(f, j * V + 8 * h + e);
            }
        }
    } else {
        // Clamped addresses keep every load in the row, so all V loads issue before one wait.
        const uint16_t* raw = reinterpret_cast<const uint16_t*>(row_start);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const int idx = j * V + e < p.experts ? j * V + e : p.experts - 1;
            const uint32_t f = static_cast<uint32_t>(raw[idx]) << 16;
            key[e] = j * V + e < p.experts ? bf16_key(f, j * V + e) : 0u;
        }
    }
}

// fp32 logits: lane j's values of logits [j V, j V + V) (padding: -inf).
template <int V>
__device__ __forceinline__ void load_row(const MoeTopkParams& p, int64_t row, int j, float (&x)[V]) {
    const float* row_start = static_cast<const float*>(p.logits) + row * p.logits_stride;
    if (p.vector_rows && p.experts == kGroupLanes * V && V >= 4) {
#pragma unroll
        for (int h = 0; h < V / 4; ++h) {
            const f32x4 v4 = *reinterpret_cast<const f32x4*>(row_start + j * V + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * h + e] = v4[e];
        }
    } else {
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const int idx = j * V + e < p.experts ? j * V + e : p.experts - 1;
            const float v = row_start[idx];
            x[e] = j * V + e < p.experts ? v : kNegInf;
        }
    }
}

template <int V>
__global__ __launch_bounds__(kMoeThreads) void moe_topk_softmax_kernel(MoeTopkParams p) {
    const int lane = threadIdx.x & 63;
    const int j = lane & (kGroupLanes - 1);
    const int64_t row = (static_cast<int64_t>(blockIdx.x) * kMoeThreads + threadIdx.x) / kGroupLanes;
    // Whole groups leave together: a group's lanes share one row (and one DPP row).
    if (row >= p.tokens) return;

    float x[V];  // this lane's logits (-inf for padding), for the all-experts normalisation
    float my_v = kNegInf, top = kNegInf;
    int my_i = 0;
    if (p.logits_is_bf16) {
        // Each lane sorts its keys once; a round takes the group's largest list head, and the lane
        // that held it (keys are unique) shifts its list by one.
        uint32_t key[V];
        load_keys<V>(p, row, j, key);
        if (p.over_all) {
#pragma unroll
            for (int e = 0; e < V; ++e) x[e] = key[e] != 0u ? key_value(key[e]) : kNegInf;
        }
        sort_desc<V>(key);
        uint32_t my_key = 0, top_key = 0;
        for (int r = 0; r < p.top_k; ++r) {
            const uint32_t best = group_max(key[0]);
            // All ones in the lane that held the winner: shift its list (a mask, not a select, so
            // the compiler keeps one operation per element).
            const uint32_t m = 0u - static_cast<uint32_t>(key[0] == best);
#pragma unroll
            for (int e = 0; e + 1 < V; ++e) key[e] = (key[e] & ~m) | (key[e + 1] & m);
            key[V - 1] &= ~m;
            my_key = j == r ? best : my_key;
            top_key = r == 0 ? best : top_key;
        }
        if (j < p.top_k) {
            my_v = key_value(my_key);
            my_i = key_expert(my_key);
        }
        top = key_value(top_key);
    } else {
        // fp32 logits: (value, index) pairs compared directly; the owning lane marks its winner.
        load_row<V>(p, row, j, x);
        uint32_t taken = 0;
#pragma unroll
        for (int e = 0; e < V; ++e) taken |= j * V + e >= p.experts ? 1u << e : 0u;
        for (int r = 0; r < p.top_k; ++r) {
            // This lane's best untaken element: indices rise with e, so a strict comparison keeps
            // the lowest index among equal values; the first candidate is taken whatever its value.
            float bv = kNegInf;
            int bi = 0x7fffffff;
            bool found = false;
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const bool take = (((taken >> e) & 1u) == 0) & (!found | (x[e] > bv));
                bv = take ? x[e] : bv;
                bi = take ? j * V + e : bi;
                found |= take;
            }
            group_best(bv, bi);
            taken |= bi / V == j ? 1u << (bi % V) : 0u;
            top = r == 0 ? bv : top;
            my_v = j == r ? bv : my_v;
            my_i = j == r ? bi : my_i;
        }
    }

    // Softmax in fp32 relative to the largest logit; no finite logit means no weight. bf16 weights
    // use the hardware exp2 and reciprocal (their error, ~1e-6 relative, is far below the bf16
    // rounding that follows); fp32 weights keep the correctly rounded expf and division.
    const bool live = top != kNegInf;
    const bool fast = p.weights_is_bf16;
    const float w_num = live && j < p.top_k ? (fast ? exp2_fast((my_v - top) * kLog2e) : expf(my_v - top)) : 0.0f;
    float denom = w_num;
    if (p.over_all) {
        denom = 0.0f;
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float d = x[e] - top;
            denom += (live & (j * V + e < p.experts)) ? (fast ? exp2_fast(d * kLog2e) : expf(d)) : 0.0f;
        }
    }
    denom = group_sum(denom);
    const float w = !live ? 0.0f : fast ? w_num * __builtin_amdgcn_rcpf(denom) : w_num / denom;

    if (j < p.top_k) {
        p.ids[row * p.ids_stride + j] = my_i;
        if (p.weights_is_bf16)
            static_cast<__bf16*>(p.weights)[row * p.weights_stride + j] = static_cast<__bf16>(w);
        else
            static_cast<float*>(p.weights)[row * p.weights_stride + j] = w;
    }
}

}  // namespace

hipError_t launch_moe_topk_softmax(const MoeTopkParams& p, hipStream_t stream) {
    const int64_t rows_per_block = kMoeThreads / kGroupLanes;
    const dim3 grid(static_cast<unsigned>((p.tokens + rows_per_block - 1) / rows_per_block));
    const int per_lane = (p.experts + kGroupLanes - 1) / kGroupLanes;
    if (per_lane <= 1)
        moe_topk_softmax_kernel<1><<<grid, dim3(kMoeThreads), 0, stream>>>(p);
    else if (per_lane <= 2)
        moe_topk_softmax_kernel<2><<<grid, dim3(kMoeThreads), 0, stream>>>(p);
    else if (per_lane <= 4)
        moe_topk_softmax_kernel<4><<<grid, dim3(kMoeThreads), 0, stream>>>(p);
    else if (per_lane <= 8)
        moe_topk_softmax_kernel<8><<<grid, dim3(kMoeThreads), 0, stream>>>(p);
    else
        moe_topk_softmax_kernel<16><<<grid, dim3(kMoeThreads), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace sinkattn
