// C ABI of libsinkattn: host-side validation and launch.
//
// Every check that needs no device access runs here, before any HIP call, so that a rejected
// call launches nothing and writes nothing. The launchers in the kernel files only size grids.

#include "sinkattn.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "launch.h"
#include "launch_ops.h"
#include "plan.h"

namespace {

thread_local std::string g_last_error;

sinkattn_status fail(sinkattn_status status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

#define SA_TRY(expr)                              \
    do {                                          \
        sinkattn_status _s = (expr);              \
        if (_s != SINKATTN_OK) return _s;         \
    } while (0)

int64_t elem_size(int32_t dt) {
    switch (dt) {
        case SINKATTN_F32: return 4;
        case SINKATTN_BF16: return 2;
        case SINKATTN_I32: return 4;
        case SINKATTN_FP8_E4M3: return 1;
    }
    return 0;
}

const char* dtype_name(int32_t dt) {
    switch (dt) {
        case SINKATTN_F32: return "f32";
        case SINKATTN_BF16: return "bf16";
        case SINKATTN_I32: return "i32";
        case SINKATTN_FP8_E4M3: return "fp8_e4m3";
    }
    return "?";
}

// Descriptor sanity: non-null, known dtype, expected rank, non-negative extents and strides.
sinkattn_status check_desc(const sinkattn_tensor* t, const char* name, int ndim) {
    if (t == nullptr) return fail(SINKATTN_ERR_NULL, "%s: descriptor is NULL", name);
    if (t->dtype != SINKATTN_F32 && t->dtype != SINKATTN_BF16 && t->dtype != SINKATTN_I32 &&
        t->dtype != SINKATTN_FP8_E4M3)
        return fail(SINKATTN_ERR_DTYPE, "%s: unknown dtype code %d", name, (int)t->dtype);
    if (t->ndim != ndim)
        return fail(SINKATTN_ERR_SHAPE, "%s: rank %d, expected %d", name, t->ndim, ndim);
    for (int i = 0; i < ndim; ++i) {
        if (t->shape[i] < 0) return fail(SINKATTN_ERR_SHAPE, "%s: negative extent", name);
        if (t->stride[i] < 0) return fail(SINKATTN_ERR_LAYOUT, "%s: negative stride", name);
    }
    return SINKATTN_OK;
}

int64_t numel(const sinkattn_tensor* t) {
    int64_t n = 1;
    for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
    return n;
}

sinkattn_status check_data(const sinkattn_tensor* t, const char* name) {
    if (numel(t) > 0 && t->data == nullptr)
        return fail(SINKATTN_ERR_NULL, "%s: data pointer is NULL", name);
    return SINKATTN_OK;
}

sinkattn_status check_dtype(const sinkattn_tensor* t, const char* name, int32_t want) {
    if (t->dtype != want)
        return fail(SINKATTN_ERR_DTYPE, "%s: dtype %s, expected %s", name, dtype_name(t->dtype),
                    dtype_name(want));
    return SINKATTN_OK;
}

// Vector-loadable rows: 16-byte aligned base, unit inner stride, outer strides multiples of
// 16 bytes. Extent-1 dimensions are never stepped, so their strides are not constrained.
sinkattn_status check_rows(const sinkattn_tensor* t, const char* name) {
    const int64_t es = elem_size(t->dtype);
    const int last = t->ndim - 1;
    if (t->stride[last] != 1 && t->shape[last] > 1)
        return fail(SINKATTN_ERR_LAYOUT, "%s: innermost stride must be 1", name);
    if (reinterpret_cast<uintptr_t>(t->data) % 16 != 0)
        return fail(SINKATTN_ERR_LAYOUT, "%s: data pointer not 16-byte aligned", name);
    for (int i = 0; i < last; ++i)
        if (t->shape[i] > 1 && (t->stride[i] * es) % 16 != 0)
            return fail(SINKATTN_ERR_LAYOUT, "%s: stride of dim %d is not a multiple of 16 bytes",
                        name, i);
    return SINKATTN_OK;
}

bool is_contiguous(const sinkattn_tensor* t) {
    int64_t expect = 1;
    for (int i = t->ndim - 1; i >= 0; --i) {
        if (t->shape[i] > 1 && t->stride[i] != expect) return false;
        expect *= t->shape[i];
    }
    return true;
}

sinkattn_status check_contiguous(const sinkattn_tensor* t, const char* name) {
    if (!is_contiguous(t)) return fail(SINKATTN_ERR_LAYOUT, "%s: must be contiguous", name);
    if (reinterpret_cast<uintptr_t>(t->data) % 16 != 0)
        return fail(SINKATTN_ERR_LAYOUT, "%s: data pointer not 16-byte aligned", name);
    return SINKATTN_OK;
}

// Writes to an output must not collide: sorted by stride, every dimension must step past the
// whole extent of the smaller ones. A tensor without elements has nothing to collide.
sinkattn_status check_no_self_overlap(const sinkattn_tensor* t, const char* name) {
    if (numel(t) == 0) return SINKATTN_OK;
    int idx[4];
    int n = 0;
    for (int i = 0; i < t->ndim; ++i)
        if (t->shape[i] > 1) idx[n++] = i;
    for (int a = 1; a < n; ++a)
        for (int b = a; b > 0 && t->stride[idx[b]] < t->stride[idx[b - 1]]; --b) {
            int tmp = idx[b];
            idx[b] = idx[b - 1];
            idx[b - 1] = tmp;
        }
    int64_t span = 1;
    for (int a = 0; a < n; ++a) {
        if (t->stride[idx[a]] < span)
            return fail(SINKATTN_ERR_LAYOUT, "%s: strides make elements overlap", name);
        span = t->stride[idx[a]] * t->shape[idx[a]];
    }
    return SINKATTN_OK;
}

struct Span {
    uintptr_t lo = 0, hi = 0;  // [lo, hi)
};

Span byte_span(const sinkattn_tensor* t) {
    Span s;
    if (t == nullptr || t->data == nullptr || numel(t) == 0) return s;
    int64_t last = 0;
    for (int i = 0; i < t->ndim; ++i) last += (t->shape[i] - 1) * t->stride[i];
    s.lo = reinterpret_cast<uintptr_t>(t->data);
    s.hi = s.lo + static_cast<uintptr_t>((last + 1) * elem_size(t->dtype));
    return s;
}

sinkattn_status check_disjoint(const sinkattn_tensor* out, const char* oname,
                               const sinkattn_tensor* in, const char* iname) {
    Span a = byte_span(out), b = byte_span(in);
    if (a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi)
        return fail(SINKATTN_ERR_LAYOUT, "%s overlaps %s", oname, iname);
    return SINKATTN_OK;
}

sinkattn_status check_scale(float scale) {
    if (!std::isfinite(scale) || !(scale > 0.0f))
        return fail(SINKATTN_ERR_SHAPE, "scale must be finite and > 0 (got %g)", (double)scale);
    return SINKATTN_OK;
}

sinkattn_status check_vec(const sinkattn_tensor* t, const char* name, sinkattn_dtype dt,
                          int64_t len) {
    SA_TRY(check_desc(t, name, 1));
    SA_TRY(check_dtype(t, name, dt));
    if (t->shape[0] != len)
        return fail(SINKATTN_ERR_SHAPE, "%s: length %lld, expected %lld", name,
                    (long long)t->shape[0], (long long)len);
    if (t->shape[0] > 1 && t->stride[0] != 1)
        return fail(SINKATTN_ERR_LAYOUT, "%s: must be contiguous", name);
    if (reinterpret_cast<uintptr_t>(t->data) % 4 != 0)
        return fail(SINKATTN_ERR_LAYOUT, "%s: data pointer not 4-byte aligned", name);
    return check_data(t, name);
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

sinkattn_status launched(hipError_t err) {
    if (err != hipSuccess)
        return fail(SINKATTN_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(err));
    return SINKATTN_OK;
}

void put_launch(sinkattn_launch& dst, const sinkattn::Launch& src) {
    static_assert(sizeof(dst.kernel) == sizeof(src.kernel), "kernel name buffers");
    memcpy(dst.kernel, src.kernel, sizeof(dst.kernel));
    dst.grid = src.grid;
    dst.block = src.block;
}

// Largest G x T query rows per KV head the multi-token decode kernel takes (four 16-column tiles).
constexpr int64_t kMaxDecodeRows = 64;

// Validation shared by the decode calls: the inputs, chunking and scale. q is [B, Hq, D], or
// [B, T, Hq, D] when `multi`. Fills the input half of `p`.
sinkattn_status check_decode_inputs(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                    const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                    const sinkattn_tensor* seqlens_k, int num_chunks, float scale,
                                    bool multi, sinkattn::DecodeSplitParams& p) {
    SA_TRY(check_desc(q, "q", multi ? 4 : 3));
    SA_TRY(check_desc(k, "k", 4));
    SA_TRY(check_desc(v, "v", 4));
    if (q->dtype != SINKATTN_BF16 && q->dtype != SINKATTN_F32)
        return fail(SINKATTN_ERR_DTYPE, "q: dtype must be bf16 or f32");
    SA_TRY(check_dtype(k, "k", q->dtype));
    SA_TRY(check_dtype(v, "v", q->dtype));

    const int qo = multi ? 1 : 0;  // q's head axis is qo + 1
    const int64_t batch = q->shape[0], q_len = multi ? q->shape[1] : 1;
    const int64_t hq = q->shape[qo + 1], dim = q->shape[qo + 2];
    const int64_t cap = k->shape[1], hkv = k->shape[2];
    for (int i = 0; i < 4; ++i)
        if (v->shape[i] != k->shape[i])
            return fail(SINKATTN_ERR_SHAPE, "v: shape differs from k");
    if (k->shape[0] != batch) return fail(SINKATTN_ERR_SHAPE, "k: batch differs from q");
    if (k->shape[3] != dim) return fail(SINKATTN_ERR_SHAPE, "k: head_dim differs from q");
    if (hkv <= 0 || hq <= 0 || hq % hkv != 0)
        return fail(SINKATTN_ERR_SHAPE, "query heads (%lld) must be a positive multiple of KV heads (%lld)",
                    (long long)hq, (long long)hkv);
    if (num_chunks < 1) return fail(SINKATTN_ERR_SHAPE, "num_chunks must be >= 1 (got %d)", num_chunks);
    SA_TRY(check_vec(seqlens_k, "seqlens_k", SINKATTN_I32, batch));
    SA_TRY(check_vec(sinks, "sinks", SINKATTN_F32, hq));
    SA_TRY(check_scale(scale));
    if (dim != sinkattn::kHeadDim)
        return fail(SINKATTN_ERR_UNSUPPORTED, "head_dim %lld not supported (only 64)", (long long)dim);
    const int64_t group = hq / hkv;
    if (!is_pow2(group) || group > 16)
        return fail(SINKATTN_ERR_UNSUPPORTED, "group size %lld not supported (1, 2, 4, 8 or 16)",
                    (long long)group);
    if (group * q_len > kMaxDecodeRows)
        return fail(SINKATTN_ERR_UNSUPPORTED,
                    "group size x tokens per sequence = %lld exceeds %lld query rows per KV head",
                    (long long)(group * q_len), (long long)kMaxDecodeRows);
    if (batch * hkv * num_chunks >= (int64_t(1) << 31) || cap >= (int64_t(1) << 31) ||
        batch * q_len * hq * num_chunks >= (int64_t(1) << 31))
        return fail(SINKATTN_ERR_UNSUPPORTED, "problem too large for one launch");
    // Cache rows of one (sequence, KV head) slice are addressed with 32-bit byte offsets,
    // including prefetches up to 512 rows past a chunk end.
    if ((cap + 512) * k->stride[1] * elem_size(k->dtype) >= (int64_t(1) << 31) ||
        (cap + 512) * v->stride[1] * elem_size(v->dtype) >= (int64_t(1) << 31))
        return fail(SINKATTN_ERR_UNSUPPORTED, "KV cache slice of one sequence exceeds 2 GiB");
    SA_TRY(check_data(q, "q"));
    SA_TRY(check_data(k, "k"));
    SA_TRY(check_data(v, "v"));
    SA_TRY(check_rows(q, "q"));
    SA_TRY(check_rows(k, "k"));
    SA_TRY(check_rows(v, "v"));

    p.q = q->data;
    p.k = k->data;
    p.v = v->data;
    p.sinks = static_cast<const float*>(sinks->data);
    p.seqlens_k = static_cast<const int32_t*>(seqlens_k->data);
    p.q_stride_b = q->stride[0];
    p.q_stride_tok = multi ? q->stride[1] : 0;
    p.q_stride_head = q->stride[qo + 1];
    p.k_stride_b = k->stride[0];
    p.k_stride_tok = k->stride[1];
    p.k_stride_head = k->stride[2];
    p.v_stride_b = v->stride[0];
    p.v_stride_tok = v->stride[1];
    p.v_stride_head = v->stride[2];
    p.capacity = cap;
    p.chunk_size = (cap + num_chunks - 1) / num_chunks;
    p.batch = static_cast<int32_t>(batch);
    p.num_q_heads = static_cast<int32_t>(hq);
    p.num_kv_heads = static_cast<int32_t>(hkv);
    p.num_chunks = num_chunks;
    p.q_len = static_cast<int32_t>(q_len);
    p.scale = scale;
    return SINKATTN_OK;
}

// Byte offsets of the fused-decode workspace regions (each 256-byte aligned).
struct WorkspaceLayout {
    size_t counters = 0, partial_o = 0, partial_m = 0, partial_d = 0, total = 0;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

WorkspaceLayout workspace_layout(int64_t batch, int64_t hq, int64_t hkv, int64_t chunks) {
    WorkspaceLayout w;
    const size_t rows = static_cast<size_t>(batch) * hq * chunks;
    w.counters = 0;
    w.partial_o = align256(static_cast<size_t>(batch) * hkv * sizeof(uint32_t));
    w.partial_m = w.partial_o + align256(rows * sinkattn::kHeadDim * sizeof(float));
    w.partial_d = w.partial_m + align256(rows * sizeof(float));
    w.total = w.partial_d + align256(rows * sizeof(float));
    return w;
}

// Validation shared by the prefill calls (everything but the outputs); fills p.
sinkattn_status check_prefill_inputs(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                     const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                     const sinkattn_tensor* cu_seqlens_q,
                                     const sinkattn_tensor* cu_seqlens_k, float scale, int causal,
                                     sinkattn::PrefillParams& p) {
    SA_TRY(check_desc(q, "q", 3));
    SA_TRY(check_desc(k, "k", 3));
    SA_TRY(check_desc(v, "v", 3));
    SA_TRY(check_desc(cu_seqlens_q, "cu_seqlens_q", 1));
    SA_TRY(check_desc(cu_seqlens_k, "cu_seqlens_k", 1));
    if (q->dtype != SINKATTN_BF16 && q->dtype != SINKATTN_F32)
        return fail(SINKATTN_ERR_DTYPE, "q: dtype must be bf16 or f32");
    SA_TRY(check_dtype(k, "k", q->dtype));
    SA_TRY(check_dtype(v, "v", q->dtype));

    const int64_t tq = q->shape[0], hq = q->shape[1], dim = q->shape[2];
    const int64_t tk = k->shape[0], hkv = k->shape[1];
    for (int i = 0; i < 3; ++i)
        if (v->shape[i] != k->shape[i])
            return fail(SINKATTN_ERR_SHAPE, "v: shape differs from k");
    if (k->shape[2] != dim) return fail(SINKATTN_ERR_SHAPE, "k: head_dim differs from q");
    if (hkv <= 0 || hq <= 0 || hq % hkv != 0)
        return fail(SINKATTN_ERR_SHAPE, "query heads (%lld) must be a positive multiple of KV heads (%lld)",
                    (long long)hq, (long long)hkv);
    if (cu_seqlens_q->shape[0] < 1 || cu_seqlens_k->shape[0] != cu_seqlens_q->shape[0])
        return fail(SINKATTN_ERR_SHAPE, "cu_seqlens_q/k must both have B+1 >= 1 entries");
    const int64_t num_seqs = cu_seqlens_q->shape[0] - 1;
    SA_TRY(check_vec(cu_seqlens_q, "cu_seqlens_q", SINKATTN_I32, num_seqs + 1));
    SA_TRY(check_vec(cu_seqlens_k, "cu_seqlens_k", SINKATTN_I32, num_seqs + 1));
    SA_TRY(check_vec(sinks, "sinks", SINKATTN_F32, hq));
    SA_TRY(check_scale(scale));
    if (dim != sinkattn::kHeadDim)
        return fail(SINKATTN_ERR_UNSUPPORTED, "head_dim %lld not supported (only 64)", (long long)dim);
    const int64_t group = hq / hkv;
    if (!is_pow2(group) || group > 128)
        return fail(SINKATTN_ERR_UNSUPPORTED, "group size %lld not supported (powers of two up to 128)",
                    (long long)group);
    if (tq >= (int64_t(1) << 31) || tk >= (int64_t(1) << 31) || num_seqs >= (int64_t(1) << 24))
        return fail(SINKATTN_ERR_UNSUPPORTED, "token or sequence count too large");
    // Key rows are addressed with 32-bit byte offsets, including prefetches up to 192 rows past
    // a sequence's end (two 64-key tiles ahead of the last one).
    if ((tk + 192) * k->stride[0] * elem_size(k->dtype) >= (int64_t(1) << 31) ||
        (tk + 192) * v->stride[0] * elem_size(v->dtype) >= (int64_t(1) << 31))
        return fail(SINKATTN_ERR_UNSUPPORTED, "K/V exceed 2 GiB of addressable rows");
    SA_TRY(check_data(q, "q"));
    SA_TRY(check_data(k, "k"));
    SA_TRY(check_data(v, "v"));
    SA_TRY(check_rows(q, "q"));
    SA_TRY(check_rows(k, "k"));
    SA_TRY(check_rows(v, "v"));

    p.q = q->data;
    p.k = k->data;
    p.v = v->data;
    p.sinks = static_cast<const float*>(sinks->data);
    p.cu_seqlens_q = static_cast<const int32_t*>(cu_seqlens_q->data);
    p.cu_seqlens_k = static_cast<const int32_t*>(cu_seqlens_k->data);
    p.q_stride_tok = q->stride[0];
    p.q_stride_head = q->stride[1];
    p.k_stride_tok = k->stride[0];
    p.k_stride_head = k->stride[1];
    p.v_stride_tok = v->stride[0];
    p.v_stride_head = v->stride[1];
    p.total_q = tq;
    p.total_k = tk;
    p.num_seqs = static_cast<int32_t>(num_seqs);
    p.num_q_heads = static_cast<int32_t>(hq);
    p.num_kv_heads = static_cast<int32_t>(hkv);
    p.scale = scale;
    p.causal = causal ? 1 : 0;
    p.num_splits = 1;
    return SINKATTN_OK;
}

// sinkattn_decode_split (q [B, Hq, D]) and sinkattn_decode_multi_split (q [B, T, Hq, D]); the
// partials of row (b, t, h) sit at (b * T + t, h), so T = 1 is the single-token layout.
sinkattn_status decode_split_impl(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                  const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                  const sinkattn_tensor* seqlens_k, int num_chunks, float scale,
                                  const sinkattn_tensor* partial_o,
                                  const sinkattn_tensor* partial_m,
                                  const sinkattn_tensor* partial_d, void* stream, bool multi) {
    g_last_error.clear();
    SA_TRY(check_desc(q, "q", multi ? 4 : 3));
    SA_TRY(check_desc(partial_o, "partial_o", 4));
    SA_TRY(check_desc(partial_m, "partial_m", 3));
    SA_TRY(check_desc(partial_d, "partial_d", 3));
    sinkattn::DecodeSplitParams p{};
    SA_TRY(check_decode_inputs(q, k, v, sinks, seqlens_k, num_chunks, scale, multi, p));
    SA_TRY(check_dtype(partial_o, "partial_o", SINKATTN_F32));
    SA_TRY(check_dtype(partial_m, "partial_m", SINKATTN_F32));
    SA_TRY(check_dtype(partial_d, "partial_d", SINKATTN_F32));
    const int64_t want_o[4] = {static_cast<int64_t>(p.batch) * p.q_len, p.num_q_heads, num_chunks,
                               sinkattn::kHeadDim};
    for (int i = 0; i < 4; ++i)
        if (partial_o->shape[i] != want_o[i])
            return fail(SINKATTN_ERR_SHAPE, multi ? "partial_o: expected [B*T, Hq, num_chunks, D]"
                                                  : "partial_o: expected [B, Hq, num_chunks, D]");
    for (int i = 0; i < 3; ++i)
        if (partial_m->shape[i] != want_o[i] || partial_d->shape[i] != want_o[i])
            return fail(SINKATTN_ERR_SHAPE, multi ? "partial_m/partial_d: expected [B*T, Hq, num_chunks]"
                                                  : "partial_m/partial_d: expected [B, Hq, num_chunks]");
    SA_TRY(check_data(partial_o, "partial_o"));
    SA_TRY(check_data(partial_m, "partial_m"));
    SA_TRY(check_data(partial_d, "partial_d"));
    SA_TRY(check_contiguous(partial_o, "partial_o"));
    SA_TRY(check_contiguous(partial_m, "partial_m"));
    SA_TRY(check_contiguous(partial_d, "partial_d"));
    const sinkattn_tensor* outs[3] = {partial_o, partial_m, partial_d};
    const char* onames[3] = {"partial_o", "partial_m", "partial_d"};
    const sinkattn_tensor* ins[5] = {q, k, v, sinks, seqlens_k};
    const char* inames[5] = {"q", "k", "v", "sinks", "seqlens_k"};
    for (int a = 0; a < 3; ++a) {
        for (int b = 0; b < 5; ++b) SA_TRY(check_disjoint(outs[a], onames[a], ins[b], inames[b]));
        for (int b = a + 1; b < 3; ++b) SA_TRY(check_disjoint(outs[a], onames[a], outs[b], onames[b]));
    }

    if (p.batch == 0 || p.q_len == 0) return SINKATTN_OK;
    p.partial_o = static_cast<float*>(partial_o->data);
    p.partial_m = static_cast<float*>(partial_m->data);
    p.partial_d = static_cast<float*>(partial_d->data);
    hipStream_t s = static_cast<hipStream_t>(stream);
    return launched(q->dtype == SINKATTN_BF16 ? sinkattn::launch_decode_split_bf16(p, s)
                                              : sinkattn::launch_decode_split_f32(p, s));
}

// sinkattn_decode (q, out [B, Hq, D], lse [B, Hq]) and sinkattn_decode_multi (q, out [B, T, Hq, D],
// lse [B, T, Hq]); the workspace holds the partials of B x T rows.
// With static_ws, the workspace is the library's own device array (sinkattn_decode_static):
// workspace/workspace_bytes are ignored and the call allocates nothing.
sinkattn_status decode_fused_impl(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                  const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                  const sinkattn_tensor* seqlens_k, int num_chunks, float scale,
                                  void* workspace, size_t workspace_bytes,
                                  const sinkattn_tensor* out, const sinkattn_tensor* lse,
                                  void* stream, bool multi, bool static_ws = false) {
    g_last_error.clear();
    const int rank = multi ? 4 : 3;
    SA_TRY(check_desc(q, "q", rank));
    SA_TRY(check_desc(out, "out", rank));
    if (lse != nullptr) SA_TRY(check_desc(lse, "lse", rank - 1));
    sinkattn::DecodeSplitParams p{};
    SA_TRY(check_decode_inputs(q, k, v, sinks, seqlens_k, num_chunks, scale, multi, p));
    if (q->dtype == SINKATTN_F32) SA_TRY(check_dtype(out, "out", SINKATTN_F32));
    else if (out->dtype != SINKATTN_BF16 && out->dtype != SINKATTN_F32)
        return fail(SINKATTN_ERR_DTYPE, "out: dtype must be bf16 or f32");
    if (lse != nullptr) SA_TRY(check_dtype(lse, "lse", SINKATTN_F32));
    for (int i = 0; i < rank; ++i)
        if (out->shape[i] != q->shape[i])
            return fail(SINKATTN_ERR_SHAPE, multi ? "out: expected [B, T, Hq, D]" : "out: expected [B, Hq, D]");
    for (int i = 0; lse != nullptr && i < rank - 1; ++i)
        if (lse->shape[i] != q->shape[i])
            return fail(SINKATTN_ERR_SHAPE, multi ? "lse: expected [B, T, Hq]" : "lse: expected [B, Hq]");
    const WorkspaceLayout w =
        workspace_layout(static_cast<int64_t>(p.batch) * p.q_len, p.num_q_heads, p.num_kv_heads, num_chunks);
    if (static_ws) {
        if (w.total > sinkattn::kStaticWorkspaceBytes)
            return fail(SINKATTN_ERR_UNSUPPORTED,
                        "chunk states need %zu bytes, more than the %zu-byte static workspace "
                        "(use sinkattn_decode with a workspace of that size)",
                        w.total, sinkattn::kStaticWorkspaceBytes);
    } else {
        if (workspace_bytes < w.total)
            return fail(SINKATTN_ERR_SHAPE, "workspace: %zu bytes, need %zu", workspace_bytes, w.total);
        if (w.total > 0 && workspace == nullptr) return fail(SINKATTN_ERR_NULL, "workspace is NULL");
        if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
            return fail(SINKATTN_ERR_LAYOUT, "workspace not 256-byte aligned");
    }
    SA_TRY(check_data(out, "out"));
    SA_TRY(check_rows(out, "out"));
    SA_TRY(check_no_self_overlap(out, "out"));
    if (lse != nullptr) {
        SA_TRY(check_data(lse, "lse"));
        if (reinterpret_cast<uintptr_t>(lse->data) % 4 != 0)
            return fail(SINKATTN_ERR_LAYOUT, "lse: data pointer not 4-byte aligned");
        if (lse->stride[rank - 2] != 1 && lse->shape[rank - 2] > 1)
            return fail(SINKATTN_ERR_LAYOUT, "lse: innermost stride must be 1");
        SA_TRY(check_no_self_overlap(lse, "lse"));
    }
    // The workspace is written too: it may not overlap any tensor argument (the static one is
    // the library's own memory, which no argument can point into).
    sinkattn_tensor ws{};
    ws.data = workspace;
    ws.dtype = SINKATTN_F32;
    ws.ndim = 1;
    ws.shape[0] = static_cast<int64_t>(w.total / 4);
    ws.stride[0] = 1;
    const sinkattn_tensor* ins[5] = {q, k, v, sinks, seqlens_k};
    const char* inames[5] = {"q", "k", "v", "sinks", "seqlens_k"};
    for (int b = 0; b < 5; ++b) {
        SA_TRY(check_disjoint(out, "out", ins[b], inames[b]));
        if (!static_ws) SA_TRY(check_disjoint(&ws, "workspace", ins[b], inames[b]));
        if (lse != nullptr) SA_TRY(check_disjoint(lse, "lse", ins[b], inames[b]));
    }
    if (!static_ws) SA_TRY(check_disjoint(out, "out", &ws, "workspace"));
    if (lse != nullptr) {
        if (!static_ws) SA_TRY(check_disjoint(lse, "lse", &ws, "workspace"));
        SA_TRY(check_disjoint(out, "out", lse, "lse"));
    }

    if (p.batch == 0 || p.q_len == 0) return SINKATTN_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (static_ws) SA_TRY(launched(sinkattn::static_decode_workspace(s, &workspace)));
    char* base = static_cast<char*>(workspace);
    p.counters = reinterpret_cast<uint32_t*>(base + w.counters);
    p.partial_o = reinterpret_cast<float*>(base + w.partial_o);
    p.partial_m = reinterpret_cast<float*>(base + w.partial_m);
    p.partial_d = reinterpret_cast<float*>(base + w.partial_d);
    p.out = out->data;
    p.lse = lse != nullptr ? static_cast<float*>(lse->data) : nullptr;
    p.o_stride_b = out->stride[0];
    p.o_stride_tok = multi ? out->stride[1] : 0;
    p.o_stride_head = out->stride[rank - 2];
    p.lse_stride_b = lse != nullptr ? lse->stride[0] : 0;
    p.lse_stride_tok = lse != nullptr && multi ? lse->stride[1] : 0;
    p.lse_stride_head = lse != nullptr ? lse->stride[rank - 2] : 0;
    p.out_is_bf16 = out->dtype == SINKATTN_BF16;
    const bool bf16 = q->dtype == SINKATTN_BF16;
    // One launch when the split grid fits a single round of work-groups; otherwise (and for the
    // fp32 reference variant) split then merge through the same workspace, which leaves the
    // arrival counters untouched.
    if (bf16 && sinkattn::decode_fused_fits_one_round(p))
        return launched(sinkattn::launch_decode_fused_bf16(p, s));
    SA_TRY(launched(bf16 ? sinkattn::launch_decode_split_bf16(p, s) : sinkattn::launch_decode_split_f32(p, s)));
    sinkattn::DecodeMergeParams mp{};
    mp.partial_o = p.partial_o;
    mp.partial_m = p.partial_m;
    mp.partial_d = p.partial_d;
    mp.out = p.out;
    mp.lse = p.lse;
    mp.o_stride_b = p.o_stride_b;
    mp.o_stride_tok = p.o_stride_tok;
    mp.o_stride_head = p.o_stride_head;
    mp.lse_stride_b = p.lse_stride_b;
    mp.lse_stride_tok = p.lse_stride_tok;
    mp.lse_stride_head = p.lse_stride_head;
    mp.batch = p.batch * p.q_len;
    mp.q_len = p.q_len;
    mp.num_q_heads = p.num_q_heads;
    mp.num_chunks = num_chunks;
    mp.out_is_bf16 = p.out_is_bf16;
    return launched(sinkattn::launch_decode_merge(mp, s));
}

// sinkattn_linear_bias (bf16) and sinkattn_linear_fp8_block_scaled (FP8 with block scales).
sinkattn_status linear_impl(const sinkattn_tensor* x, const sinkattn_tensor* scale_x,
                            const sinkattn_tensor* w, const sinkattn_tensor* scale_w,
                            const sinkattn_tensor* bias, const sinkattn_tensor* y, void* stream, bool fp8) {
    g_last_error.clear();
    SA_TRY(check_desc(x, "x", 2));
    SA_TRY(check_desc(w, "w", 2));
    SA_TRY(check_desc(y, "y", 2));
    if (bias != nullptr) SA_TRY(check_desc(bias, "bias", 1));
    if (fp8) {
        SA_TRY(check_desc(scale_x, "scale_x", 2));
        SA_TRY(check_desc(scale_w, "scale_w", 2));
    }
    const sinkattn_dtype in = fp8 ? SINKATTN_FP8_E4M3 : SINKATTN_BF16;
    SA_TRY(check_dtype(x, "x", in));
    SA_TRY(check_dtype(w, "w", in));
    if (y->dtype != SINKATTN_BF16 && y->dtype != SINKATTN_F32)
        return fail(SINKATTN_ERR_DTYPE, "y: dtype must be bf16 or f32");
    if (bias != nullptr) SA_TRY(check_dtype(bias, "bias", SINKATTN_F32));
    if (fp8) {
        SA_TRY(check_dtype(scale_x, "scale_x", SINKATTN_F32));
        SA_TRY(check_dtype(scale_w, "scale_w", SINKATTN_F32));
    }
    const int64_t m = x->shape[0], k = x->shape[1], n = w->shape[0];
    const int64_t step = fp8 ? 128 : 64;
    if (w->shape[1] != k) return fail(SINKATTN_ERR_SHAPE, "w: expected [N, K] with the K of x");
    if (y->shape[0] != m || y->shape[1] != n) return fail(SINKATTN_ERR_SHAPE, "y: expected [M, N]");
    if (bias != nullptr && bias->shape[0] != n) return fail(SINKATTN_ERR_SHAPE, "bias: expected [N]");
    if (k <= 0 || k % step != 0)
        return fail(SINKATTN_ERR_SHAPE, "K (%lld) must be a positive multiple of %lld", (long long)k,
                    (long long)step);
    if (fp8) {
        if (scale_x->shape[0] != m || scale_x->shape[1] != k / 128)
            return fail(SINKATTN_ERR_SHAPE, "scale_x: expected [M, K/128]");
        if (scale_w->shape[0] != (n + 127) / 128 || scale_w->shape[1] != k / 128)
            return fail(SINKATTN_ERR_SHAPE, "scale_w: expected [ceil(N/128), K/128]");
    }
    const int64_t es = elem_size(in);
    if (m >= (int64_t(1) << 31) || n >= (int64_t(1) << 31) ||
        ((m + 127) / 128) * ((n + 127) / 128) >= (int64_t(1) << 31))
        return fail(SINKATTN_ERR_UNSUPPORTED, "problem too large for one launch");
    // A work-group addresses its (up to 256) rows of x and of w with 32-bit byte offsets.
    if (256 * x->stride[0] * es >= (int64_t(1) << 31) || 256 * w->stride[0] * es >= (int64_t(1) << 31))
        return fail(SINKATTN_ERR_UNSUPPORTED, "row stride too large (256 rows must span < 2 GiB)");
    SA_TRY(check_data(x, "x"));
    SA_TRY(check_data(w, "w"));
    SA_TRY(check_data(y, "y"));
    if (bias != nullptr) SA_TRY(check_data(bias, "bias"));
    if (fp8) {
        SA_TRY(check_data(scale_x, "scale_x"));
        SA_TRY(check_data(scale_w, "scale_w"));
    }
    SA_TRY(check_rows(x, "x"));
    SA_TRY(check_rows(w, "w"));
    if ((m > 1 && x->stride[0] < k) || (n > 1 && w->stride[0] < k))
        return fail(SINKATTN_ERR_LAYOUT, "x/w: rows overlap (row stride below K)");
    if (bias != nullptr && bias->stride[0] != 1 && n > 1)
        return fail(SINKATTN_ERR_LAYOUT, "bias: must be contiguous");
    if (y->stride[1] != 1 && n > 1) return fail(SINKATTN_ERR_LAYOUT, "y: innermost stride must be 1");
    const sinkattn_tensor* aligned[4] = {bias, y, scale_x, scale_w};
    const char* anames[4] = {"bias", "y", "scale_x", "scale_w"};
    for (int a = 0; a < 4; ++a)
        if (aligned[a] != nullptr && reinterpret_cast<uintptr_t>(aligned[a]->data) % elem_size(aligned[a]->dtype) != 0)
            return fail(SINKATTN_ERR_LAYOUT, "%s: data pointer not element-aligned", anames[a]);
    SA_TRY(check_no_self_overlap(y, "y"));
    const sinkattn_tensor* ins[5] = {x, w, bias, scale_x, scale_w};
    const char* inames[5] = {"x", "w", "bias", "scale_x", "scale_w"};
    for (int b = 0; b < 5; ++b)
        if (ins[b] != nullptr) SA_TRY(check_disjoint(y, "y", ins[b], inames[b]));

    if (m == 0 || n == 0) return SINKATTN_OK;
    sinkattn::GemmParams p{};
    p.x = x->data;
    p.w = w->data;
    p.bias = bias != nullptr ? static_cast<const float*>(bias->data) : nullptr;
    p.y = y->data;
    p.scale_x = fp8 ? static_cast<const float*>(scale_x->data) : nullptr;
    p.scale_w = fp8 ? static_cast<const float*>(scale_w->data) : nullptr;
    // A single row's stride is never stepped: the buffer range then spans just its K elements.
    p.ldx = m > 1 ? x->stride[0] : k;
    p.ldw = n > 1 ? w->stride[0] : k;
    p.ldy = y->stride[0];
    p.sx_stride_m = fp8 ? scale_x->stride[0] : 0;
    p.sx_stride_kb = fp8 ? scale_x->stride[1] : 0;
    p.sw_stride_nb = fp8 ? scale_w->stride[0] : 0;
    p.sw_stride_kb = fp8 ? scale_w->stride[1] : 0;
    p.m = static_cast<int32_t>(m);
    p.n = static_cast<int32_t>(n);
    p.k = static_cast<int32_t>(k);
    p.y_is_bf16 = y->dtype == SINKATTN_BF16;
    return launched(sinkattn::launch_gemm_bias(p, fp8, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

sinkattn_status sinkattn_prefill(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                 const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                 const sinkattn_tensor* cu_seqlens_q,
                                 const sinkattn_tensor* cu_seqlens_k, float scale, int causal,
                                 const sinkattn_tensor* out, void* stream) {
    g_last_error.clear();
    SA_TRY(check_desc(out, "out", 3));
    sinkattn::PrefillParams p{};
    SA_TRY(check_prefill_inputs(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, scale, causal, p));
    if (q->dtype == SINKATTN_F32) SA_TRY(check_dtype(out, "out", SINKATTN_F32));
    else if (out->dtype != SINKATTN_BF16 && out->dtype != SINKATTN_F32)
        return fail(SINKATTN_ERR_DTYPE, "out: dtype must be bf16 or f32");
    for (int i = 0; i < 3; ++i)
        if (out->shape[i] != q->shape[i])
            return fail(SINKATTN_ERR_SHAPE, "out: shape differs from q");
    SA_TRY(check_data(out, "out"));
    SA_TRY(check_rows(out, "out"));
    SA_TRY(check_no_self_overlap(out, "out"));
    SA_TRY(check_disjoint(out, "out", q, "q"));
    SA_TRY(check_disjoint(out, "out", k, "k"));
    SA_TRY(check_disjoint(out, "out", v, "v"));
    SA_TRY(check_disjoint(out, "out", sinks, "sinks"));
    SA_TRY(check_disjoint(out, "out", cu_seqlens_q, "cu_seqlens_q"));
    SA_TRY(check_disjoint(out, "out", cu_seqlens_k, "cu_seqlens_k"));

    if (p.total_q == 0 || p.num_seqs == 0) return SINKATTN_OK;
    p.out = out->data;
    p.o_stride_tok = out->stride[0];
    p.o_stride_head = out->stride[1];
    p.out_is_bf16 = out->dtype == SINKATTN_BF16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return launched(q->dtype == SINKATTN_BF16 ? sinkattn::launch_prefill_bf16(p, s)
                                              : sinkattn::launch_prefill_f32(p, s));
}

sinkattn_status sinkattn_prefill_split(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                       const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                       const sinkattn_tensor* cu_seqlens_q,
                                       const sinkattn_tensor* cu_seqlens_k, float scale,
                                       int causal, int num_splits,
                                       const sinkattn_tensor* partial_o,
                                       const sinkattn_tensor* partial_m,
                                       const sinkattn_tensor* partial_d, void* stream) {
    g_last_error.clear();
    SA_TRY(check_desc(partial_o, "partial_o", 4));
    SA_TRY(check_desc(partial_m, "partial_m", 3));
    SA_TRY(check_desc(partial_d, "partial_d", 3));
    sinkattn::PrefillParams p{};
    SA_TRY(check_prefill_inputs(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, scale, causal, p));
    if (num_splits < 1 || num_splits > 65536)
        return fail(SINKATTN_ERR_SHAPE, "num_splits must be in [1, 65536] (got %d)", num_splits);
    SA_TRY(check_dtype(partial_o, "partial_o", SINKATTN_F32));
    SA_TRY(check_dtype(partial_m, "partial_m", SINKATTN_F32));
    SA_TRY(check_dtype(partial_d, "partial_d", SINKATTN_F32));
    const int64_t want_o[4] = {q->shape[0], q->shape[1], num_splits, q->shape[2]};
    for (int i = 0; i < 4; ++i)
        if (partial_o->shape[i] != want_o[i])
            return fail(SINKATTN_ERR_SHAPE, "partial_o: expected [Tq, Hq, num_splits, D]");
    for (int i = 0; i < 3; ++i)
        if (partial_m->shape[i] != want_o[i] || partial_d->shape[i] != want_o[i])
            return fail(SINKATTN_ERR_SHAPE, "partial_m/partial_d: expected [Tq, Hq, num_splits]");
    if (p.total_q * p.num_q_heads * static_cast<int64_t>(num_splits) >= (int64_t(1) << 31))
        return fail(SINKATTN_ERR_UNSUPPORTED, "Tq * Hq * num_splits too large");
    SA_TRY(check_data(partial_o, "partial_o"));
    SA_TRY(check_data(partial_m, "partial_m"));
    SA_TRY(check_data(partial_d, "partial_d"));
    SA_TRY(check_contiguous(partial_o, "partial_o"));
    SA_TRY(check_contiguous(partial_m, "partial_m"));
    SA_TRY(check_contiguous(partial_d, "partial_d"));
    const sinkattn_tensor* outs[3] = {partial_o, partial_m, partial_d};
    const char* onames[3] = {"partial_o", "partial_m", "partial_d"};
    const sinkattn_tensor* ins[6] = {q, k, v, sinks, cu_seqlens_q, cu_seqlens_k};
    const char* inames[6] = {"q", "k", "v", "sinks", "cu_seqlens_q", "cu_seqlens_k"};
    for (int a = 0; a < 3; ++a) {
        for (int b = 0; b < 6; ++b) SA_TRY(check_disjoint(outs[a], onames[a], ins[b], inames[b]));
        for (int b = a + 1; b < 3; ++b) SA_TRY(check_disjoint(outs[a], onames[a], outs[b], onames[b]));
    }

    if (p.total_q == 0 || p.num_seqs == 0) return SINKATTN_OK;
    p.num_splits = num_splits;
    p.partial_o = static_cast<float*>(partial_o->data);
    p.partial_m = static_cast<float*>(partial_m->data);
    p.partial_d = static_cast<float*>(partial_d->data);
    hipStream_t s = static_cast<hipStream_t>(stream);
    return launched(q->dtype == SINKATTN_BF16 ? sinkattn::launch_prefill_bf16(p, s)
                                              : sinkattn::launch_prefill_f32(p, s));
}

sinkattn_status sinkattn_decode_split(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                      const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                      const sinkattn_tensor* seqlens_k, int num_chunks,
                                      float scale, const sinkattn_tensor* partial_o,
                                      const sinkattn_tensor* partial_m,
                                      const sinkattn_tensor* partial_d, void* stream) {
    return decode_split_impl(q, k, v, sinks, seqlens_k, num_chunks, scale, partial_o, partial_m,
                             partial_d, stream, false);
}

sinkattn_status sinkattn_decode_multi_split(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                            const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                            const sinkattn_tensor* seqlens_k, int num_chunks,
                                            float scale, const sinkattn_tensor* partial_o,
                                            const sinkattn_tensor* partial_m,
                                            const sinkattn_tensor* partial_d, void* stream) {
    return decode_split_impl(q, k, v, sinks, seqlens_k, num_chunks, scale, partial_o, partial_m,
                             partial_d, stream, true);
}

sinkattn_status sinkattn_decode(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                const sinkattn_tensor* seqlens_k, int num_chunks, float scale,
                                void* workspace, size_t workspace_bytes,
                                const sinkattn_tensor* out, const sinkattn_tensor* lse,
                                void* stream) {
    return decode_fused_impl(q, k, v, sinks, seqlens_k, num_chunks, scale, workspace,
                             workspace_bytes, out, lse, stream, false);
}

sinkattn_status sinkattn_decode_multi(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                      const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                      const sinkattn_tensor* seqlens_k, int num_chunks, float scale,
                                      void* workspace, size_t workspace_bytes,
                                      const sinkattn_tensor* out, const sinkattn_tensor* lse,
                                      void* stream) {
    return decode_fused_impl(q, k, v, sinks, seqlens_k, num_chunks, scale, workspace,
                             workspace_bytes, out, lse, stream, true);
}

sinkattn_status sinkattn_decode_static(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                       const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                       const sinkattn_tensor* seqlens_k, int num_chunks, float scale,
                                       const sinkattn_tensor* out, const sinkattn_tensor* lse,
                                       void* stream) {
    static_assert(SINKATTN_DECODE_STATIC_WORKSPACE_BYTES == sinkattn::kStaticWorkspaceBytes,
                  "header and library agree on the static workspace size");
    return decode_fused_impl(q, k, v, sinks, seqlens_k, num_chunks, scale, nullptr, 0, out, lse, stream,
                             /*multi=*/false, /*static_ws=*/true);
}

size_t sinkattn_decode_workspace_size(int64_t batch, int64_t num_q_heads, int64_t num_kv_heads,
                                      int num_chunks) {
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_chunks < 1) return 0;
    return workspace_layout(batch, num_q_heads, num_kv_heads, num_chunks).total;
}

size_t sinkattn_decode_workspace_counter_bytes(int64_t batch, int64_t num_kv_heads) {
    if (batch < 0 || num_kv_heads <= 0) return 0;
    return align256(static_cast<size_t>(batch) * num_kv_heads * sizeof(uint32_t));
}

sinkattn_status sinkattn_decode_merge(const sinkattn_tensor* partial_o,
                                      const sinkattn_tensor* partial_m,
                                      const sinkattn_tensor* partial_d, int num_chunks,
                                      const sinkattn_tensor* out, const sinkattn_tensor* lse,
                                      void* stream) {
    g_last_error.clear();
    SA_TRY(check_desc(partial_o, "partial_o", 4));
    SA_TRY(check_desc(partial_m, "partial_m", 3));
    SA_TRY(check_desc(partial_d, "partial_d", 3));
    SA_TRY(check_desc(out, "out", 3));
    if (lse != nullptr) SA_TRY(check_desc(lse, "lse", 2));
    SA_TRY(check_dtype(partial_o, "partial_o", SINKATTN_F32));
    SA_TRY(check_dtype(partial_m, "partial_m", SINKATTN_F32));
    SA_TRY(check_dtype(partial_d, "partial_d", SINKATTN_F32));
    if (out->dtype != SINKATTN_BF16 && out->dtype != SINKATTN_F32)
        return fail(SINKATTN_ERR_DTYPE, "out: dtype must be bf16 or f32");
    if (lse != nullptr) SA_TRY(check_dtype(lse, "lse", SINKATTN_F32));

    const int64_t batch = partial_o->shape[0], hq = partial_o->shape[1];
    const int64_t chunks = partial_o->shape[2], dim = partial_o->shape[3];
    if (num_chunks < 1 || num_chunks != chunks)
        return fail(SINKATTN_ERR_SHAPE, "num_chunks (%d) must equal the chunk extent of partial_o (%lld)",
                    num_chunks, (long long)chunks);
    for (int i = 0; i < 3; ++i)
        if (partial_m->shape[i] != partial_o->shape[i] || partial_d->shape[i] != partial_o->shape[i])
            return fail(SINKATTN_ERR_SHAPE, "partial_m/partial_d: expected [B, Hq, num_chunks]");
    if (out->shape[0] != batch || out->shape[1] != hq || out->shape[2] != dim)
        return fail(SINKATTN_ERR_SHAPE, "out: expected [B, Hq, D]");
    if (lse != nullptr && (lse->shape[0] != batch || lse->shape[1] != hq))
        return fail(SINKATTN_ERR_SHAPE, "lse: expected [B, Hq]");
    if (dim != sinkattn::kHeadDim)
        return fail(SINKATTN_ERR_UNSUPPORTED, "head_dim %lld not supported (only 64)", (long long)dim);
    if (batch * hq >= (int64_t(1) << 31))
        return fail(SINKATTN_ERR_UNSUPPORTED, "problem too large for one launch");

    SA_TRY(check_data(partial_o, "partial_o"));
    SA_TRY(check_data(partial_m, "partial_m"));
    SA_TRY(check_data(partial_d, "partial_d"));
    SA_TRY(check_data(out, "out"));
    if (lse != nullptr) {
        SA_TRY(check_data(lse, "lse"));
        if (reinterpret_cast<uintptr_t>(lse->data) % 4 != 0)
            return fail(SINKATTN_ERR_LAYOUT, "lse: data pointer not 4-byte aligned");
        if (lse->stride[1] != 1 && lse->shape[1] > 1)
            return fail(SINKATTN_ERR_LAYOUT, "lse: innermost stride must be 1");
        SA_TRY(check_no_self_overlap(lse, "lse"));
    }
    SA_TRY(check_contiguous(partial_o, "partial_o"));
    SA_TRY(check_contiguous(partial_m, "partial_m"));
    SA_TRY(check_contiguous(partial_d, "partial_d"));
    SA_TRY(check_rows(out, "out"));
    SA_TRY(check_no_self_overlap(out, "out"));
    const sinkattn_tensor* ins[3] = {partial_o, partial_m, partial_d};
    const char* inames[3] = {"partial_o", "partial_m", "partial_d"};
    for (int b = 0; b < 3; ++b) {
        SA_TRY(check_disjoint(out, "out", ins[b], inames[b]));
        if (lse != nullptr) SA_TRY(check_disjoint(lse, "lse", ins[b], inames[b]));
    }
    if (lse != nullptr) SA_TRY(check_disjoint(out, "out", lse, "lse"));

    if (batch == 0 || hq == 0) return SINKATTN_OK;

    sinkattn::DecodeMergeParams p{};
    p.partial_o = static_cast<const float*>(partial_o->data);
    p.partial_m = static_cast<const float*>(partial_m->data);
    p.partial_d = static_cast<const float*>(partial_d->data);
    p.out = out->data;
    p.lse = lse != nullptr ? static_cast<float*>(lse->data) : nullptr;
    p.o_stride_b = out->stride[0];
    p.o_stride_head = out->stride[1];
    p.lse_stride_b = lse != nullptr ? lse->stride[0] : 0;
    p.lse_stride_head = lse != nullptr ? lse->stride[1] : 0;
    p.batch = static_cast<int32_t>(batch);
    p.q_len = 1;
    p.num_q_heads = static_cast<int32_t>(hq);
    p.num_chunks = num_chunks;
    p.out_is_bf16 = out->dtype == SINKATTN_BF16;
    return launched(sinkattn::launch_decode_merge(p, static_cast<hipStream_t>(stream)));
}

sinkattn_status sinkattn_moe_topk_softmax(const sinkattn_tensor* logits, int top_k, int over_all_experts,
                                          const sinkattn_tensor* topk_ids,
                                          const sinkattn_tensor* topk_weights, void* stream) {
    g_last_error.clear();
    SA_TRY(check_desc(logits, "logits", 2));
    SA_TRY(check_desc(topk_ids, "topk_ids", 2));
    SA_TRY(check_desc(topk_weights, "topk_weights", 2));
    if (logits->dtype != SINKATTN_BF16 && logits->dtype != SINKATTN_F32)
        return fail(SINKATTN_ERR_DTYPE, "logits: dtype must be bf16 or f32");
    SA_TRY(check_dtype(topk_ids, "topk_ids", SINKATTN_I32));
    if (topk_weights->dtype != SINKATTN_BF16 && topk_weights->dtype != SINKATTN_F32)
        return fail(SINKATTN_ERR_DTYPE, "topk_weights: dtype must be bf16 or f32");
    const int64_t tokens = logits->shape[0], experts = logits->shape[1];
    if (top_k < 1) return fail(SINKATTN_ERR_SHAPE, "top_k must be >= 1 (got %d)", top_k);
    if (topk_ids->shape[0] != tokens || topk_ids->shape[1] != top_k)
        return fail(SINKATTN_ERR_SHAPE, "topk_ids: expected [T, top_k]");
    if (topk_weights->shape[0] != tokens || topk_weights->shape[1] != top_k)
        return fail(SINKATTN_ERR_SHAPE, "topk_weights: expected [T, top_k]");
    if (experts < 1 || top_k > experts)
        return fail(SINKATTN_ERR_SHAPE, "top_k (%d) must not exceed the expert count (%lld)", top_k,
                    (long long)experts);
    if (experts > 256 || top_k > 16)
        return fail(SINKATTN_ERR_UNSUPPORTED, "at most 256 experts and top_k <= 16 (got %lld, %d)",
                    (long long)experts, top_k);
    if (tokens >= (int64_t(1) << 35))
        return fail(SINKATTN_ERR_UNSUPPORTED, "problem too large for one launch");
    SA_TRY(check_data(logits, "logits"));
    SA_TRY(check_data(topk_ids, "topk_ids"));
    SA_TRY(check_data(topk_weights, "topk_weights"));
    if (logits->stride[1] != 1 && experts > 1)
        return fail(SINKATTN_ERR_LAYOUT, "logits: innermost stride must be 1");
    if (reinterpret_cast<uintptr_t>(logits->data) % elem_size(logits->dtype) != 0)
        return fail(SINKATTN_ERR_LAYOUT, "logits: data pointer not element-aligned");
    const sinkattn_tensor* outs[2] = {topk_ids, topk_weights};
    const char* onames[2] = {"topk_ids", "topk_weights"};
    for (int a = 0; a < 2; ++a) {
        if (outs[a]->stride[1] != 1 && outs[a]->shape[1] > 1)
            return fail(SINKATTN_ERR_LAYOUT, "%s: innermost stride must be 1", onames[a]);
        if (reinterpret_cast<uintptr_t>(outs[a]->data) % elem_size(outs[a]->dtype) != 0)
            return fail(SINKATTN_ERR_LAYOUT, "%s: data pointer not element-aligned", onames[a]);
        SA_TRY(check_no_self_overlap(outs[a], onames[a]));
        SA_TRY(check_disjoint(outs[a], onames[a], logits, "logits"));
    }
    SA_TRY(check_disjoint(topk_ids, "topk_ids", topk_weights, "topk_weights"));

    if (tokens == 0) return SINKATTN_OK;
    sinkattn::MoeTopkParams p{};
    p.logits = logits->data;
    p.ids = static_cast<int32_t*>(topk_ids->data);
    p.weights = topk_weights->data;
    p.logits_stride = logits->stride[0];
    p.ids_stride = topk_ids->stride[0];
    p.weights_stride = topk_weights->stride[0];
    p.tokens = tokens;
    p.experts = static_cast<int32_t>(experts);
    p.top_k = top_k;
    p.over_all = over_all_experts != 0;
    p.logits_is_bf16 = logits->dtype == SINKATTN_BF16;
    p.weights_is_bf16 = topk_weights->dtype == SINKATTN_BF16;
    // 16-byte row loads only where every row starts on a 16-byte boundary.
    p.vector_rows = reinterpret_cast<uintptr_t>(logits->data) % 16 == 0 &&
                    (tokens == 1 || (logits->stride[0] * elem_size(logits->dtype)) % 16 == 0);
    return launched(sinkattn::launch_moe_topk_softmax(p, static_cast<hipStream_t>(stream)));
}

sinkattn_status sinkattn_linear_bias(const sinkattn_tensor* x, const sinkattn_tensor* w,
                                     const sinkattn_tensor* bias, const sinkattn_tensor* y,
                                     void* stream) {
    return linear_impl(x, nullptr, w, nullptr, bias, y, stream, false);
}

sinkattn_status sinkattn_linear_fp8_block_scaled(const sinkattn_tensor* x, const sinkattn_tensor* scale_x,
                                                 const sinkattn_tensor* w, const sinkattn_tensor* scale_w,
                                                 const sinkattn_tensor* bias, const sinkattn_tensor* y,
                                                 void* stream) {
    return linear_impl(x, scale_x, w, scale_w, bias, y, stream, true);
}

const char* sinkattn_status_string(sinkattn_status status) {
    switch (status) {
        case SINKATTN_OK: return "ok";
        case SINKATTN_ERR_NULL: return "null pointer";
        case SINKATTN_ERR_DTYPE: return "unsupported or mismatched dtype";
        case SINKATTN_ERR_SHAPE: return "inconsistent shape or bad argument";
        case SINKATTN_ERR_LAYOUT: return "unsupported memory layout";
        case SINKATTN_ERR_UNSUPPORTED: return "unsupported configuration";
        case SINKATTN_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

const char* sinkattn_last_error(void) { return g_last_error.c_str(); }

sinkattn_status sinkattn_plan_decode(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                     const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                     const sinkattn_tensor* seqlens_k, int num_chunks, float scale,
                                     int form, sinkattn_launch* launches, int* count) {
    g_last_error.clear();
    if (launches == nullptr || count == nullptr) return fail(SINKATTN_ERR_NULL, "launches/count is NULL");
    *count = 0;
    if (form != SINKATTN_PLAN_DECODE_SPLIT && form != SINKATTN_PLAN_DECODE)
        return fail(SINKATTN_ERR_SHAPE, "unknown plan form %d", form);
    if (q == nullptr) return fail(SINKATTN_ERR_NULL, "q is NULL");
    const bool multi = q->ndim == 4;
    sinkattn::DecodeSplitParams p{};
    SA_TRY(check_decode_inputs(q, k, v, sinks, seqlens_k, num_chunks, scale, multi, p));
    if (p.batch == 0 || p.q_len == 0) return SINKATTN_OK;
    const bool bf16 = q->dtype == SINKATTN_BF16;
    if (form == SINKATTN_PLAN_DECODE && bf16 && sinkattn::decode_fused_fits_one_round(p)) {
        put_launch(launches[0], sinkattn::plan_decode_split_bf16(p, true));
        *count = 1;
        return SINKATTN_OK;
    }
    put_launch(launches[0], bf16 ? sinkattn::plan_decode_split_bf16(p, false) : sinkattn::plan_decode_split_f32(p));
    *count = 1;
    if (form == SINKATTN_PLAN_DECODE) {
        sinkattn::DecodeMergeParams mp{};
        mp.batch = p.batch * p.q_len;
        mp.q_len = p.q_len;
        mp.num_q_heads = p.num_q_heads;
        mp.num_chunks = num_chunks;
        put_launch(launches[1], sinkattn::plan_decode_merge(mp));
        *count = 2;
    }
    return SINKATTN_OK;
}

sinkattn_status sinkattn_plan_prefill(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                      const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                      const sinkattn_tensor* cu_seqlens_q,
                                      const sinkattn_tensor* cu_seqlens_k, float scale, int causal,
                                      int num_splits, sinkattn_launch* launches, int* count) {
    g_last_error.clear();
    if (launches == nullptr || count == nullptr) return fail(SINKATTN_ERR_NULL, "launches/count is NULL");
    *count = 0;
    sinkattn::PrefillParams p{};
    SA_TRY(check_prefill_inputs(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, scale, causal, p));
    if (num_splits < 0 || num_splits > 65536)
        return fail(SINKATTN_ERR_SHAPE, "num_splits must be 0 (unsplit) or in [1, 65536] (got %d)", num_splits);
    if (num_splits > 0 && p.total_q * p.num_q_heads * static_cast<int64_t>(num_splits) >= (int64_t(1) << 31))
        return fail(SINKATTN_ERR_UNSUPPORTED, "Tq * Hq * num_splits too large");
    if (p.total_q == 0 || p.num_seqs == 0) return SINKATTN_OK;
    // The launchers tell the split form by a non-null partial_o; the plan only needs that bit.
    static float split_marker;
    if (num_splits > 0) {
        p.num_splits = num_splits;
        p.partial_o = &split_marker;
    }
    const sinkattn::Launch l =
        q->dtype == SINKATTN_BF16 ? sinkattn::plan_prefill_bf16(p) : sinkattn::plan_prefill_f32(p);
    if (l.grid > sinkattn::kMaxGrid) return fail(SINKATTN_ERR_UNSUPPORTED, "problem too large for one launch");
    put_launch(launches[0], l);
    *count = 1;
    return SINKATTN_OK;
}

int sinkattn_version(void) { return SINKATTN_VERSION; }

}  // extern "C"
