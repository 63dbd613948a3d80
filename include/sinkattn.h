/*
 * sinkattn.h - C ABI of libsinkattn: grouped-query attention with a learned per-head softmax sink,
 * and the MoE routing softmax and bias / FP8 block-scaled linear layers of the same model,
 * hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * The operation (blog post "GPT-OSS on Day 0", Perplexity, 2025; section "Kernels for GPT-OSS",
 * subsection "Sink attention"): every query head h owns one learned scalar sink[h]. For a query
 * row q the attention weights are the softmax over the scaled logits scale * <q, k_j> of the keys
 * the row may see, extended by one extra logit equal to sink[h]. The sink column has no value
 * vector: it only adds e^(sink[h]) to the softmax denominator, so
 *
 *     out = sum_j e^(s_j) v_j / ( e^(sink[h]) + sum_j e^(s_j) ),   s_j = scale * <q, k_j>.
 *
 * The kernels compute this with the online softmax described in the same subsection: a running
 * maximum m and running scale d per row, with m started at the head's sink value and d at 1 (the
 * sink's own term). When the KV sequence is split into chunks, the sink is folded into the first
 * chunk only (chunk 0) and the chunks are combined by a log-sum-exp merge.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensors are passed as sinkattn_tensor descriptors: a device pointer, an element type, a rank
 *    and per-dimension extents and strides (strides in elements). The innermost dimension must have
 *    stride 1. Data pointers must be 16-byte aligned and every non-inner stride a multiple of
 *    8 elements (bf16) or 4 elements (fp32), so rows can be moved with 128-bit loads.
 *  - head_dim D must be 64. Hq must be a multiple of Hkv; query head h reads KV head h / (Hq/Hkv)
 *    (contiguous groups).
 *  - q, k, v (and out) are either all bf16 (the MFMA fast path) or all fp32 (the reference
 *    variant). With bf16 inputs `out` may be bf16 or fp32. Softmax state and accumulation are fp32.
 *  - The library allocates nothing, frees nothing, never synchronises the stream and never reads
 *    device memory on the host. Every call is stateless and reentrant; work is enqueued on
 *    `stream` (a hipStream_t; NULL means the default stream).
 *  - Outputs must not overlap inputs (checked on the host from the descriptors).
 *  - All checks that can be made on the host run before any launch. On any error nothing is
 *    launched and nothing is written; the status says which class of error it was, and
 *    sinkattn_last_error() returns a message for the calling thread. A launch the HIP runtime
 *    rejects returns SINKATTN_ERR_LAUNCH. Faults inside kernels surface at the caller's next
 *    synchronisation, like any HIP kernel.
 *  - Device-side preconditions (documented, not checked, since checking them would need a device
 *    read): cu_seqlens are non-decreasing, start at 0 and end at the token counts; seqlens_k[b] is
 *    in [0, Lcap]. Kernels clamp indices so that a broken precondition cannot read or write out
 *    of the tensors' bounds; the values computed are then unspecified.
 */
#ifndef SINKATTN_H
#define SINKATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SINKATTN_VERSION 7

typedef enum {
    SINKATTN_OK = 0,
    SINKATTN_ERR_NULL = 1,        /* a required descriptor or data pointer is NULL */
    SINKATTN_ERR_DTYPE = 2,       /* element type not allowed for this argument, or mismatched */
    SINKATTN_ERR_SHAPE = 3,       /* wrong rank, inconsistent extents, bad scalar argument */
    SINKATTN_ERR_LAYOUT = 4,      /* misaligned pointer, non-unit inner stride, bad stride, overlap */
    SINKATTN_ERR_UNSUPPORTED = 5, /* well-formed but not implemented (e.g. head_dim != 64) */
    SINKATTN_ERR_LAUNCH = 6       /* the HIP runtime rejected a kernel launch */
} sinkattn_status;

typedef enum {
    SINKATTN_F32 = 0,
    SINKATTN_BF16 = 1,
    SINKATTN_I32 = 2,
    SINKATTN_FP8_E4M3 = 3 /* OCP E4M3 (1-4-3, bias 7, no infinities), one byte per element */
} sinkattn_dtype;

/* A strided view of device memory. Only the first `ndim` entries of shape/stride are read. */
typedef struct {
    void* data;          /* device pointer (caller-owned) */
    int32_t dtype;       /* a sinkattn_dtype value; any other value is rejected (SINKATTN_ERR_DTYPE) */
    int32_t ndim;        /* 1..4 */
    int64_t shape[4];    /* extents, >= 0 */
    int64_t stride[4];   /* in elements */
} sinkattn_tensor;

/*
 * sinkattn_prefill - causal (or full) varlen prefill over a packed batch of B sequences.
 *
 * Source: "GPT-OSS on Day 0", "Sink attention" subsection: the sink-attention formula, evaluated
 * with the online softmax whose running max starts at the head's sink. One work-group walks every
 * KV tile of its query rows, so the sink is folded once per row, before the first tile.
 *
 *   q            [Tq, Hq, D]   bf16 | fp32   packed queries of all sequences
 *   k, v         [Tk, Hkv, D]  same dtype as q
 *   sinks        [Hq]          fp32          learned sink logit per query head (finite or -inf;
 *                                            it is NOT multiplied by `scale`)
 *   cu_seqlens_q [B+1]         int32 device  prefix sums of query lengths (cu[0] = 0, cu[B] = Tq)
 *   cu_seqlens_k [B+1]         int32 device  prefix sums of key lengths   (cu[B] = Tk)
 *   scale        finite, > 0 (typically 1/sqrt(D))
 *   causal       nonzero: query i of a sequence with Lq queries and Lk keys sees keys
 *                j <= i + (Lk - Lq) (bottom-right aligned; with Lq = Lk the usual j <= i).
 *                zero: every query sees every key of its sequence.
 *   out          [Tq, Hq, D]   bf16 | fp32 (fp32 only if q is fp32)
 *
 * A row that sees no key returns 0 (all weight sits on the value-less sink; with sink = -inf the
 * 0/0 row is defined as 0). Tq = 0 or B = 0 launches nothing and returns SINKATTN_OK.
 * Supported group sizes Hq/Hkv: powers of two up to 128.
 */
sinkattn_status sinkattn_prefill(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                 const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                 const sinkattn_tensor* cu_seqlens_q,
                                 const sinkattn_tensor* cu_seqlens_k, float scale, int causal,
                                 const sinkattn_tensor* out, void* stream);

/*
 * sinkattn_prefill_split - varlen prefill split along each sequence's KV length.
 *
 * Source: "GPT-OSS on Day 0", "Sink attention" subsection: when attention is split into chunks
 * along the KV length, the sink is folded into the first chunk only; the same rule applied to
 * prefill. Meant for prefills whose query tiles alone cannot fill the GPU (a few hundred new tokens
 * against a long cache): each (query tile, KV head, split) is its own work-group. The partials
 * use the decode format, and sinkattn_decode_merge with partial_o viewed as [Tq, Hq, S, D]
 * ("batch" = Tq) combines them into the sinkattn_prefill result (equal up to rounding).
 *
 *   q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, scale, causal: as for sinkattn_prefill
 *   num_splits   S >= 1. Split j of sequence b covers its keys [j*ks, min((j+1)*ks, Lk_b)),
 *                ks = ceil(Lk_b / S) rounded up to a multiple of 64; splits past the end are empty.
 *   partial_o    [Tq, Hq, S, D] fp32 contiguous   o = the split's softmax-weighted mean of V
 *   partial_m    [Tq, Hq, S]    fp32 contiguous   m = a reference logit of the split (natural log)
 *   partial_d    [Tq, Hq, S]    fp32 contiguous   d = sum of e^(term - m) over the split's terms
 * A row's state in a split covers the keys of the split it may see (causal rule as above), plus
 * the sink in split 0. A split with no such term is (o, m, d) = (0, -inf, 0).
 */
sinkattn_status sinkattn_prefill_split(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                       const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                       const sinkattn_tensor* cu_seqlens_q,
                                       const sinkattn_tensor* cu_seqlens_k, float scale,
                                       int causal, int num_splits,
                                       const sinkattn_tensor* partial_o,
                                       const sinkattn_tensor* partial_m,
                                       const sinkattn_tensor* partial_d, void* stream);

/*
 * sinkattn_decode_split - one query token per sequence against a padded KV cache, split along the
 * KV length into `num_chunks` chunks of cs = ceil(Lcap / num_chunks) keys.
 *
 * Source: "GPT-OSS on Day 0", "Sink attention" subsection: attention is parallelised over heads
 * and over KV length, and the sink is counted in the first chunk only. Chunk c of sequence b
 * covers keys [c*cs, min((c+1)*cs, seqlens_k[b])); chunk 0 always carries the sink, even when it
 * holds no key. For every (b, query head h, chunk c) the call writes the chunk's softmax state:
 *
 *   partial_m[b,h,c] = m_c, the largest logit of the chunk (with the sink for c = 0), natural log;
 *   partial_d[b,h,c] = d_c = sum over the chunk's terms of e^(term - m_c);
 *   partial_o[b,h,c,:] = (sum_j e^(s_j - m_c) v_j) / d_c, the chunk's normalised output.
 *
 * An empty chunk c >= 1 writes m = -inf, d = 0, o = 0. Only (m_c + ln d_c) and o_c are
 * determined by the mathematics; m_c may differ from the exact maximum by rounding.
 *
 *   q          [B, Hq, D]          bf16 | fp32
 *   k, v       [B, Lcap, Hkv, D]   same dtype as q; rows at or past seqlens_k[b] are never read
 *   sinks      [Hq]                fp32
 *   seqlens_k  [B]                 int32 device, each in [0, Lcap]
 *   num_chunks C >= 1
 *   scale      finite, > 0
 *   partial_o  [B, Hq, C, D] fp32, contiguous
 *   partial_m, partial_d [B, Hq, C] fp32, contiguous
 *
 * Supported group sizes Hq/Hkv: 1, 2, 4, 8, 16. B = 0 launches nothing.
 */
sinkattn_status sinkattn_decode_split(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                      const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                      const sinkattn_tensor* seqlens_k, int num_chunks,
                                      float scale, const sinkattn_tensor* partial_o,
                                      const sinkattn_tensor* partial_m,
                                      const sinkattn_tensor* partial_d, void* stream);

/*
 * sinkattn_decode_merge - log-sum-exp merge of the chunk states written by sinkattn_decode_split.
 *
 * Source: the chunk combination that the "Sink attention" subsection's split along the KV length
 * requires (the page describes the split and the first-chunk rule, not the combination; this is
 * the standard log-sum-exp merge of softmax states). Per (b, h):
 *
 *   M = max_c m_c,  w_c = d_c e^(m_c - M) (0 when m_c = -inf),
 *   out = sum_c w_c o_c / sum_c w_c,  lse = M + ln sum_c w_c.
 *
 * The sink is counted once because only chunk 0 carries it. If every chunk is empty and the sink
 * is -inf, out = 0 and lse = -inf.
 *
 *   partial_o  [B, Hq, C, D] fp32, contiguous
 *   partial_m, partial_d [B, Hq, C] fp32, contiguous
 *   num_chunks C, must equal the chunk extent of the partials
 *   out        [B, Hq, D] bf16 | fp32
 *   lse        [B, Hq] fp32 or NULL (not written)
 */
sinkattn_status sinkattn_decode_merge(const sinkattn_tensor* partial_o,
                                      const sinkattn_tensor* partial_m,
                                      const sinkattn_tensor* partial_d, int num_chunks,
                                      const sinkattn_tensor* out, const sinkattn_tensor* lse,
                                      void* stream);

/*
 * sinkattn_decode - split-KV decode and its log-sum-exp merge, through one workspace.
 *
 * Same computation and inputs as sinkattn_decode_split followed by sinkattn_decode_merge ("GPT-OSS
 * on Day 0", "Sink attention" subsection: split along the KV length, sink in the first chunk only,
 * chunks combined). When the bf16 split grid has at most one work-group per compute unit it runs
 * as one launch: every work-group writes its chunk states into `workspace`, counts itself done on
 * a per-(sequence, KV-head group) counter, and the last one to finish merges that group's chunks
 * and writes `out` (and `lse`). Larger grids, and fp32 inputs, run the split and the merge as two
 * launches on `stream` through the same workspace (the counters are not touched). Both forms
 * compute the same quantities; their merges may round differently in the last bits.
 *
 *   q, k, v, sinks, seqlens_k, num_chunks, scale: as for sinkattn_decode_split
 *   workspace       device memory, 256-byte aligned, at least
 *                   sinkattn_decode_workspace_size(B, Hq, Hkv, num_chunks) bytes. Its counter
 *                   region (the first sinkattn_decode_workspace_counter_bytes(B, Hkv) bytes) must
 *                   be zero before the first call (e.g. one hipMemsetAsync after allocating);
 *                   every call that runs to completion leaves it zero again, so a workspace can be
 *                   reused, also by calls replayed from a HIP graph. Calls sharing a workspace must
 *                   not overlap in time.
 *   workspace_bytes size of that memory
 *   out             [B, Hq, D] bf16 | fp32 (fp32 only if q is fp32)
 *   lse             [B, Hq] fp32 (natural log of each row's softmax denominator) or NULL
 *
 * Supported group sizes Hq/Hkv: 1, 2, 4, 8, 16. B = 0 launches nothing.
 */
sinkattn_status sinkattn_decode(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                const sinkattn_tensor* seqlens_k, int num_chunks, float scale,
                                void* workspace, size_t workspace_bytes,
                                const sinkattn_tensor* out, const sinkattn_tensor* lse,
                                void* stream);

/*
 * sinkattn_decode_multi_split - T new tokens per sequence (speculative or multi-token
 * verification) against the padded KV cache that already holds them, split along the KV length.
 *
 * Source: "GPT-OSS on Day 0", "Sink attention" subsection, as for sinkattn_decode_split (heads and
 * KV length in parallel, sink in the first chunk only), for the T last rows of a causal sequence:
 * with L = seqlens_k[b] keys (the T new tokens included), token t of sequence b sees keys
 * j <= L - T + t (the causal rule of sinkattn_prefill for Lq = T, Lk = L). The G = Hq/Hkv heads
 * and T tokens that share a KV head are computed together, so the cache is read once for all of
 * them.
 *
 *   q          [B, T, Hq, D]       bf16 | fp32
 *   k, v, sinks, seqlens_k, num_chunks, scale: as for sinkattn_decode_split (chunk c covers keys
 *              [c*cs, (c+1)*cs), cs = ceil(Lcap / num_chunks), each token clipped to its own limit;
 *              chunk 0 always carries the sink)
 *   partial_o  [B*T, Hq, C, D] fp32, contiguous  (row b*T + t holds token t of sequence b)
 *   partial_m, partial_d [B*T, Hq, C] fp32, contiguous
 * The states follow sinkattn_decode_split's definition per (b, t, h, c); sinkattn_decode_merge on
 * these partials with out viewed as [B*T, Hq, D] gives the attention outputs. Supported: group
 * sizes 1, 2, 4, 8, 16 with G * T <= 64. B = 0 or T = 0 launches nothing.
 */
sinkattn_status sinkattn_decode_multi_split(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                            const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                            const sinkattn_tensor* seqlens_k, int num_chunks,
                                            float scale, const sinkattn_tensor* partial_o,
                                            const sinkattn_tensor* partial_m,
                                            const sinkattn_tensor* partial_d, void* stream);
/*
 * sinkattn_decode_multi - sinkattn_decode_multi_split and the merge through one workspace, as
 * sinkattn_decode does for one token.
 *
 *   q               [B, T, Hq, D] bf16 | fp32
 *   workspace       as for sinkattn_decode, sized by sinkattn_decode_workspace_size(B * T, Hq, Hkv,
 *                   num_chunks), with its first sinkattn_decode_workspace_counter_bytes(B * T, Hkv)
 *                   bytes zero before the first call (left zero by every completed call)
 *   out             [B, T, Hq, D] bf16 | fp32 (fp32 only if q is fp32)
 *   lse             [B, T, Hq] fp32 or NULL
 * Other arguments and limits as for sinkattn_decode_multi_split.
 */
sinkattn_status sinkattn_decode_multi(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                      const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                      const sinkattn_tensor* seqlens_k, int num_chunks, float scale,
                                      void* workspace, size_t workspace_bytes,
                                      const sinkattn_tensor* out, const sinkattn_tensor* lse,
                                      void* stream);
/*
 * sinkattn_decode_static - sinkattn_decode without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. The call allocates nothing (no hipMalloc, no allocating library routine).
 *
 * The chunk states and arrival counters live in a device array owned by the library,
 * SINKATTN_DECODE_STATIC_WORKSPACE_BYTES bytes on each GPU it runs on, held from the time the
 * library's code is loaded until the process ends. The first call on a device (the current one)
 * looks its address up and clears it with one kernel on `stream`, ahead of the call's own kernels;
 * every completed call leaves its counters zero again. All calls on one GPU share that array, so
 * calls that overlap in time on one GPU (other streams, other host threads) race and give wrong
 * results; serialise them.
 *
 * Arguments, results and limits as for sinkattn_decode (one token per sequence), plus: a problem
 * whose chunk states need more than SINKATTN_DECODE_STATIC_WORKSPACE_BYTES
 * (sinkattn_decode_workspace_size(B, Hq, Hkv, num_chunks) bytes) returns SINKATTN_ERR_UNSUPPORTED
 * before anything is launched. B = 0 launches nothing and does not touch the device.
 */
#define SINKATTN_DECODE_STATIC_WORKSPACE_BYTES ((size_t)32 << 20)
sinkattn_status sinkattn_decode_static(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                       const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                       const sinkattn_tensor* seqlens_k, int num_chunks, float scale,
                                       const sinkattn_tensor* out, const sinkattn_tensor* lse,
                                       void* stream);

/* Bytes of workspace sinkattn_decode needs (0 for invalid arguments). */
size_t sinkattn_decode_workspace_size(int64_t batch, int64_t num_q_heads, int64_t num_kv_heads,
                                      int num_chunks);

/* Bytes at the start of that workspace holding the counters that must start at zero. */
size_t sinkattn_decode_workspace_counter_bytes(int64_t batch, int64_t num_kv_heads);

/*
 * sinkattn_moe_topk_softmax - MoE routing weights: the top-K experts of every token and a softmax
 * taken over the K chosen logits only.
 *
 * Source: "GPT-OSS on Day 0" (Perplexity): the model outline ("GPT-OSS on Hopper") lists a softmax
 * after the top-K choice for the expert weights; section "Kernels for GPT-OSS" says the routing
 * scores take the softmax over the top-K chosen experts only, unlike DeepSeek-style models that
 * take it over all experts, and that computing the expert weights in bfloat16 matters for accuracy.
 *
 *   logits        [T, E]  bf16 | fp32   router logits (finite or -inf; no NaN), unit inner stride
 *   top_k         K, 1 <= K <= min(E, 16); E <= 256
 *   over_all_experts  zero: weights = softmax over the K chosen logits (each row sums to 1);
 *                 nonzero: softmax over all E logits, the K chosen entries of it (the contrast mode)
 *   topk_ids      [T, K] int32   chosen experts, by logit descending; among equal logits the lower
 *                                expert index comes first
 *   topk_weights  [T, K] bf16 | fp32   computed in fp32, stored rounded to nearest (bf16)
 * A row whose largest logit is -inf gets weights 0. T = 0 launches nothing.
 */
sinkattn_status sinkattn_moe_topk_softmax(const sinkattn_tensor* logits, int top_k, int over_all_experts,
                                          const sinkattn_tensor* topk_ids,
                                          const sinkattn_tensor* topk_weights, void* stream);
/*
 * sinkattn_linear_bias - linear layer y = x w^T + bias, bf16, with the bias folded into the
 * matrix-core accumulators.
 *
 * Source: "GPT-OSS on Day 0" (Perplexity): the GEMM kernels were extended with a bias term
 * ("GPT-OSS on Hopper"), added by starting the accumulator registers at bias values loaded from
 * memory once per output block ("Kernels for GPT-OSS"). Every output tile's accumulators start at
 * the bias of their column; no separate epilogue pass reads the bias.
 *
 *   x     [M, K] bf16   activations, unit inner stride, rows 16-byte aligned
 *   w     [N, K] bf16   weights (as a linear layer stores them), same layout rules
 *   bias  [N] fp32, contiguous, or NULL (no bias)
 *   y     [M, N] bf16 | fp32, unit inner stride; must not overlap the inputs
 * K must be a positive multiple of 64. Accumulation is fp32. M = 0 or N = 0 launches nothing.
 */
sinkattn_status sinkattn_linear_bias(const sinkattn_tensor* x, const sinkattn_tensor* w,
                                     const sinkattn_tensor* bias, const sinkattn_tensor* y,
                                     void* stream);
/*
 * sinkattn_linear_fp8_block_scaled - linear layer y = dequant(x) dequant(w)^T + bias with FP8 (E4M3)
 * operands and 128 x 128 block scaling, bias folded into the accumulators.
 *
 * Source: "GPT-OSS on Day 0" (Perplexity), section "GPT-OSS on Hopper": FP8 with 128x128 block
 * scaling as the quantisation scheme, GEMM kernels extended with a bias; "Kernels for GPT-OSS":
 * the accumulators start at the bias. The pages scale the weights in 128 x 128 blocks and do not
 * say how the activations are scaled; here x carries one scale per row and 128-column block:
 *
 *   y[m, n] = bias[n] + sum_kb scale_x[m, kb] * scale_w[n / 128, kb] * sum_{k in block kb} x[m, k] w[n, k]
 *
 *   x        [M, K] FP8_E4M3, unit inner stride, rows 16-byte aligned
 *   scale_x  [M, K/128] fp32 (any strides)
 *   w        [N, K] FP8_E4M3, unit inner stride, rows 16-byte aligned
 *   scale_w  [ceil(N/128), K/128] fp32 (any strides)
 *   bias     [N] fp32, contiguous, or NULL
 *   y        [M, N] bf16 | fp32, unit inner stride
 * K must be a positive multiple of 128. Each 128-wide k block is multiplied exactly (FP8 products
 * accumulate in fp32) and added to the fp32 accumulator times its two scales. NaN codes propagate.
 */
sinkattn_status sinkattn_linear_fp8_block_scaled(const sinkattn_tensor* x, const sinkattn_tensor* scale_x,
                                                 const sinkattn_tensor* w, const sinkattn_tensor* scale_w,
                                                 const sinkattn_tensor* bias, const sinkattn_tensor* y,
                                                 void* stream);
/* ---------------------------------------------------------------------------------------------
 * Launch plans: the kernels a call launches for given inputs, reported without launching.
 *
 * For profilers and reports (which kernel of a profile belongs to which call) and for checking
 * the grid choice on a machine without a GPU. The inputs are validated exactly as the call itself
 * validates them (same status and sinkattn_last_error text on rejection); their data pointers are
 * checked for alignment only and never dereferenced, so host addresses or placeholders of the
 * right alignment do. Nothing is launched, allocated or synchronised.
 *
 *   kernel   the kernel's name as a profiler prints it, without namespace or parameter list
 *            (template arguments included, e.g. "decode_split_bf16_kernel<2, false, true, true>")
 *   grid     work-groups of the launch
 *   block    threads per work-group
 */
typedef struct {
    char kernel[96];
    int64_t grid;
    int32_t block;
} sinkattn_launch;

/* Which call of the decode family to plan (the `form` argument of sinkattn_plan_decode). */
typedef enum {
    SINKATTN_PLAN_DECODE_SPLIT = 0, /* sinkattn_decode_split (q rank 3) / _multi_split (q rank 4) */
    SINKATTN_PLAN_DECODE = 1        /* sinkattn_decode / _multi / _static (same kernels) */
} sinkattn_plan_form;

/* Plans of the decode family for q [B, Hq, D] or [B, T, Hq, D], k/v, sinks, seqlens_k, num_chunks
 * and scale as in those calls. Writes the launches in launch order to launches[0 .. *count - 1]:
 * one for the split form; for sinkattn_decode one (split and merge in a single launch) or two
 * (split, then merge); none when B = 0 or T = 0. `launches` must have room for two entries.
 * Section "Kernels for GPT-OSS", subsection "Sink attention", of "GPT-OSS on Day 0" (the
 * split-KV decode these kernels carry out). */
sinkattn_status sinkattn_plan_decode(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                     const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                     const sinkattn_tensor* seqlens_k, int num_chunks, float scale,
                                     int form, sinkattn_launch* launches, int* count);

/* Plan of sinkattn_prefill (num_splits = 0) or sinkattn_prefill_split (num_splits >= 1) for
 * these inputs: one launch in launches[0], none when Tq = 0 or B = 0. */
sinkattn_status sinkattn_plan_prefill(const sinkattn_tensor* q, const sinkattn_tensor* k,
                                      const sinkattn_tensor* v, const sinkattn_tensor* sinks,
                                      const sinkattn_tensor* cu_seqlens_q,
                                      const sinkattn_tensor* cu_seqlens_k, float scale, int causal,
                                      int num_splits, sinkattn_launch* launches, int* count);

/* Short static description of a status code. Never NULL. */
const char* sinkattn_status_string(sinkattn_status status);

/* Detail of the last error reported on the calling thread ("" if none). Valid until the thread's
 * next sinkattn call. */
const char* sinkattn_last_error(void);

/* SINKATTN_VERSION of the built library. */
int sinkattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SINKATTN_H */
