// Host-only stand-ins for the kernel launchers of libsinkattn, for checking the C-ABI layer
// (api.cpp) on a machine without a GPU, under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// api.cpp is compiled unchanged and linked against this file instead of the HIP kernel files.
// Every launcher records what it was asked to launch -- the kernel, grid and work-group size the
// shared launch plans (plan.h) give for its parameters, and the parameters the kernel would read --
// as one line of JSON, and launches nothing. Tests read the lines back through
// sinkattn_stub_take_log and can make the next launcher report a HIP error
// (sinkattn_stub_fail_next) to exercise the launch-failure path.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "launch.h"
#include "launch_ops.h"
#include "plan.h"

namespace {

std::mutex g_mutex;
std::string g_log;
hipError_t g_fail_next = hipSuccess;

void append(const std::string& line) {
    std::lock_guard<std::mutex> lock(g_mutex);
    g_log += line;
    g_log += '\n';
}

hipError_t take_status() {
    std::lock_guard<std::mutex> lock(g_mutex);
    const hipError_t e = g_fail_next;
    g_fail_next = hipSuccess;
    return e;
}

std::string fmt(const char* f, ...) __attribute__((format(printf, 1, 2)));
std::string fmt(const char* f, ...) {
    char buf[1024];
    va_list ap;
    va_start(ap, f);
    vsnprintf(buf, sizeof(buf), f, ap);
    va_end(ap);
    return buf;
}

unsigned long long addr(const void* p) { return static_cast<unsigned long long>(reinterpret_cast<uintptr_t>(p)); }

std::string launch_fields(const sinkattn::Launch& l) {
    return fmt("\"kernel\": \"%s\", \"grid\": %lld, \"block\": %d", l.kernel, static_cast<long long>(l.grid), l.block);
}

hipError_t record_decode(const char* launcher, const sinkattn::DecodeSplitParams& p, const sinkattn::Launch& l) {
    const sinkattn::DecodeShape s = sinkattn::decode_shape(p);
    append(fmt("{\"launcher\": \"%s\", %s, \"heads_per_group\": %d, \"key_split\": %s, \"private_staging\": %s, \"batch\": %d, "
               "\"q_len\": %d, \"num_q_heads\": %d, \"num_kv_heads\": %d, \"num_chunks\": %d, "
               "\"capacity\": %lld, \"chunk_size\": %lld, \"k_stride_head\": %lld, \"partial_o\": %llu, "
               "\"partial_m\": %llu, \"partial_d\": %llu, \"counters\": %llu, \"out\": %llu, \"lse\": %llu, "
               "\"out_is_bf16\": %d}",
               launcher, launch_fields(l).c_str(), s.heads, s.key_split ? "true" : "false", s.private_staging ? "true" : "false", p.batch, p.q_len,
               p.num_q_heads, p.num_kv_heads, p.num_chunks, static_cast<long long>(p.capacity),
               static_cast<long long>(p.chunk_size), static_cast<long long>(p.k_stride_head), addr(p.partial_o),
               addr(p.partial_m), addr(p.partial_d), addr(p.counters), addr(p.out), addr(p.lse), p.out_is_bf16));
    return take_status();
}

hipError_t record_prefill(const char* launcher, const sinkattn::PrefillParams& p, const sinkattn::Launch& l) {
    const sinkattn::PrefillShape s = sinkattn::prefill_shape(p);
    if (l.grid > sinkattn::kMaxGrid) return hipErrorInvalidConfiguration;
    append(fmt("{\"launcher\": \"%s\", %s, \"positions_per_tile\": %d, \"tiles\": %lld, \"total_q\": %lld, "
               "\"total_k\": %lld, \"num_seqs\": %d, \"num_q_heads\": %d, \"num_kv_heads\": %d, \"num_splits\": %d, "
               "\"causal\": %d, \"out_is_bf16\": %d}",
               launcher, launch_fields(l).c_str(), s.positions_per_tile, static_cast<long long>(s.tiles),
               static_cast<long long>(p.total_q), static_cast<long long>(p.total_k), p.num_seqs, p.num_q_heads,
               p.num_kv_heads, p.num_splits, p.causal, p.out_is_bf16));
    return take_status();
}

}  // namespace

namespace sinkattn {

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t) {
    return record_prefill("prefill_bf16", p, plan_prefill_bf16(p));
}

hipError_t launch_prefill_f32(const PrefillParams& p, hipStream_t) {
    return record_prefill("prefill_f32", p, plan_prefill_f32(p));
}

hipError_t launch_decode_split_bf16(const DecodeSplitParams& p, hipStream_t) {
    return record_decode("decode_split_bf16", p, plan_decode_split_bf16(p, false));
}

hipError_t launch_decode_split_f32(const DecodeSplitParams& p, hipStream_t) {
    return record_decode("decode_split_f32", p, plan_decode_split_f32(p));
}

hipError_t launch_decode_fused_bf16(const DecodeSplitParams& p, hipStream_t) {
    return record_decode("decode_fused_bf16", p, plan_decode_split_bf16(p, true));
}

hipError_t launch_decode_merge(const DecodeMergeParams& p, hipStream_t) {
    const Launch l = plan_decode_merge(p);
    append(fmt("{\"launcher\": \"decode_merge\", %s, \"batch\": %d, \"q_len\": %d, \"num_q_heads\": %d, "
               "\"num_chunks\": %d, \"partial_o\": %llu, \"partial_m\": %llu, \"partial_d\": %llu, \"out\": %llu, "
               "\"lse\": %llu, \"o_stride_b\": %lld, \"o_stride_tok\": %lld, \"o_stride_head\": %lld, "
               "\"out_is_bf16\": %d}",
               launch_fields(l).c_str(), p.batch, p.q_len, p.num_q_heads, p.num_chunks, addr(p.partial_o),
               addr(p.partial_m), addr(p.partial_d), addr(p.out), addr(p.lse), static_cast<long long>(p.o_stride_b),
               static_cast<long long>(p.o_stride_tok), static_cast<long long>(p.o_stride_head), p.out_is_bf16));
    return take_status();
}

hipError_t launch_moe_topk_softmax(const MoeTopkParams& p, hipStream_t) {
    append(fmt("{\"launcher\": \"moe_topk\", \"tokens\": %lld, \"experts\": %d, \"top_k\": %d, \"over_all\": %d, "
               "\"vector_rows\": %d}",
               static_cast<long long>(p.tokens), p.experts, p.top_k, p.over_all, p.vector_rows));
    return take_status();
}

hipError_t launch_gemm_bias(const GemmParams& p, bool fp8, hipStream_t) {
    append(fmt("{\"launcher\": \"gemm\", \"m\": %d, \"n\": %d, \"k\": %d, \"fp8\": %s, \"bias\": %s}", p.m, p.n,
               p.k, fp8 ? "true" : "false", p.bias != nullptr ? "true" : "false"));
    return take_status();
}

// The static workspace's device address stands in as a fixed, 256-byte aligned placeholder.
constexpr uintptr_t kStubStaticWorkspace = uintptr_t(0x7e00) << 32;

hipError_t static_decode_workspace(hipStream_t, void** out) {
    *out = reinterpret_cast<void*>(kStubStaticWorkspace);
    append(fmt("{\"launcher\": \"static_workspace\", \"address\": %llu}",
               static_cast<unsigned long long>(kStubStaticWorkspace)));
    return hipSuccess;
}

}  // namespace sinkattn

extern "C" {

// The HIP runtime is not linked: the one runtime call api.cpp makes is this one, on its error path.
const char* hipGetErrorString(hipError_t error) {
    switch (error) {
        case hipSuccess: return "no error (stub)";
        case hipErrorInvalidConfiguration: return "invalid configuration (stub)";
        case hipErrorLaunchFailure: return "launch failure (stub)";
        default: return "error (stub)";
    }
}

// Copies the records logged since the last call (one JSON object per line) into buf (NUL-ended,
// truncated to n - 1 bytes) and clears them; returns the full length of the records.
size_t sinkattn_stub_take_log(char* buf, size_t n) {
    std::lock_guard<std::mutex> lock(g_mutex);
    const size_t len = g_log.size();
    if (buf != nullptr && n > 0) {
        const size_t k = len < n - 1 ? len : n - 1;
        memcpy(buf, g_log.data(), k);
        buf[k] = '\0';
    }
    g_log.clear();
    return len;
}

// The next launcher called reports `error` (a hipError_t value) after recording its launch.
void sinkattn_stub_fail_next(int error) {
    std::lock_guard<std::mutex> lock(g_mutex);
    g_fail_next = static_cast<hipError_t>(error);
}

}  // extern "C"
