/*
 * ua.h -- C ABI of the unified paged, variable-length attention forward for
 * AMD Instinct MI355X (gfx950).
 *
 * One call computes, for a batch of sequences whose query tokens are packed
 * back to back, softmax(q K^T * scale) V against a paged KV cache, per query
 * head, with grouped-query heads, a causal or full mask, and an optional split
 * of the key range into partial results merged by a log-sum-exp combine.
 *
 * Where each operation is defined (citations are to the pages this library
 * implements):
 *   - the attention itself: page "flashatten takeaways EP2 工程", section
 *     "kv cache", the boxed formula O = softmax(q K^T / sqrt(d)) V over every
 *     cached token;
 *   - packed queries, cu_seqlens_q, the paged cache layout [num_blocks,
 *     block_size, kv_heads, head_size] with its four strides, per-sequence
 *     block tables, num_queries_per_kv = Hq / Hkv, context_len and the fp8
 *     dequantisation scales: page "vLLM Triton unified attention notes",
 *     sections test_triton_unified_attn, unified_attention and
 *     kernel_unified_attention_2d;
 *   - the split-KV partial pass and the combine that corrects the partials:
 *     page "flashatten takeaways EP2 工程", section "源代码接口" (the
 *     run_flash_splitkv_fwd interface and its combine launch, at most 128
 *     splits); page "Fused Attention", section FlashDecoding;
 *   - the log-sum-exp of each output row: page "Fused Attention", the
 *     tutorial's forward epilogue (m += log2 l, stored per row).
 *
 * Conventions shared by every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     allocates no memory, keeps no mutable global state and is thread-safe.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it: no host synchronisation, no device-to-host copy.
 *   - Element strides are in elements, not bytes; the innermost (head_size)
 *     stride is always 1.
 *   - Host-checkable violations return a negative ua_status and enqueue
 *     nothing.  Data-dependent violations (q_len > kv_len, a block id outside
 *     [0, num_blocks), max_seqlen_* smaller than the true maximum, a
 *     cu_seqlens_q that is not non-decreasing) are undefined behaviour and are
 *     not checked on the device.
 */
#ifndef UA_H
#define UA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define UA_ABI_VERSION 5u

typedef enum {
    UA_OK = 0,
    UA_ERR_INVALID_ARG = -1,   /* null pointer, bad size, stride or alignment, abi mismatch */
    UA_ERR_UNSUPPORTED = -2,   /* valid but not implemented: head_size != 128, fp8 q, ... */
    UA_ERR_WORKSPACE = -3,     /* num_splits > 1 without a large enough workspace */
    UA_ERR_HIP = -4,           /* the HIP runtime refused a launch */
    UA_ERR_SCRATCH = -5        /* ua_unified_attention_noalloc: partials exceed its scratch */
} ua_status;

typedef enum {
    UA_BF16 = 0,               /* bfloat16 */
    UA_FP16 = 1,               /* IEEE binary16 */
    UA_FP8_E4M3FN = 2          /* OCP 8-bit E4M3FN (bias 7, max 448, no inf); KV cache only */
} ua_dtype;

/*
 * Arguments of one attention call.  Start from ua_attn_params_init(): a
 * zero-filled struct is not the default, since window_left = window_right = 0
 * asks for a local window of the query's own key.  Shapes use
 *   S = num_seqs, T = num_tokens, Hq = num_q_heads, Hkv = num_kv_heads,
 *   D = head_size, NB = num_blocks, bs = block_size, W = block_table_stride.
 *
 * q            [T, Hq, D] of q_dtype (bf16 or fp16); token t of sequence s is
 *              row cu_seqlens_q[s] + i, i < q_len(s).  Strides q_stride_token,
 *              q_stride_head.
 * k_cache,     [NB, bs, Hkv, D] of kv_dtype (q_dtype, or fp8 e4m3fn).  Both
 * v_cache      caches use the strides kv_stride_block, kv_stride_slot,
 *              kv_stride_head.  Key position j of sequence s lives in physical
 *              block block_table[s * W + j / bs], slot j % bs.
 * out          [T, Hq, D] of q_dtype; strides o_stride_token, o_stride_head.
 *              Rows of tokens that belong to no sequence (tokens at or past
 *              cu_seqlens_q[S], padding) are not written, with or without
 *              splits.
 * cu_seqlens_q [S + 1] int32, cu_seqlens_q[0] = 0, non-decreasing; q_len(s) =
 *              cu[s + 1] - cu[s] (0 allowed); cu[S] <= T.
 * seqused_k    [S] int32: kv_len(s), the number of keys of sequence s, which
 *              includes its q_len(s) new tokens (kv_len >= q_len).
 * block_table  [S, W] int32 physical block ids; entries at or past
 *              ceil(kv_len(s) / bs) are never read (they may hold anything).
 * max_seqlen_q, max_seqlen_k  caller-guaranteed upper bounds of q_len and
 *              kv_len (they size the launch on the host).
 * softmax_scale  finite and > 0 (scores are scale * q . k).
 * causal       0: every query sees keys [0, kv_len).  1: query i of sequence
 *              s sits at position kv_len - q_len + i and sees keys
 *              [0, kv_len - q_len + i] (queries are the newest tokens).
 * window_left, local attention (the window switches of the FA2 forward launch,
 * window_right page "flashatten takeaways EP2 工程", section "源代码接口"): the
 *              query at position pos = kv_len - q_len + i also needs
 *              pos - window_left <= j (window_left >= 0) and
 *              j <= pos + window_right (window_right >= 0); -1 = no bound on
 *              that side.  Combined with causal, causal is the tighter right
 *              bound.
 * alibi_slopes optional [Hq] device fp32 (4-byte aligned), or NULL: ALiBi (the
 *              same launch's alibi_slopes_ptr switch).  The logit of key j for
 *              query head h is softmax_scale * q . k_j - alibi_slopes[h] *
 *              |pos - j|.  Positions must stay below 2^24 (exact in fp32).
 * fp8_compute  0 or 1; 1 needs an fp8 cache and no window / ALiBi (else
 *              UA_ERR_UNSUPPORTED).  Sequences with q_len * (Hq / Hkv) > 32
 *              query rows then run on the fp8 matrix cores (the fp8 attention
 *              variants of page "flashatten takeaways EP2 工程", section
 *              "源代码接口"): each query row (token, head) is rounded to e4m3 as
 *              code = rne(clamp(q / s, -448, 448)) with s = max|q_row| / 448
 *              in fp32 (s = 1 for an all-zero row).  The softmax weights
 *              w_j = 2^(x_j - m) (x the row's scores in log2 units) are
 *              taken against a per-row running reference m: the maximum of
 *              the first 64-key tile that holds a visible key, moved to a
 *              later tile's maximum only when that exceeds m by more than 8
 *              (so w_j <= 2^8), each key group and split keeping its own; each
 *              w_j is rounded to the nearest e4m3fn value (ties to even,
 *              subnormals k * 2^-9 kept) before P V, while the row sum adds
 *              the unrounded weights.  When a row's keys fit one tile, its
 *              output is sum_j e4m3(w_j) v_j / sum_j w_j with m the row's
 *              maximum.  Shorter sequences keep the 16-bit path.  Results
 *              differ from fp8_compute = 0 by these roundings.
 * k_scale,     device fp32 scalars (4-byte aligned), required iff kv_dtype is
 * v_scale      fp8 (else NULL): a stored code c means the value c * scale.
 * num_splits   0 = choose automatically, 1 = no split, 2..128 = split each
 *              query block's key range into that many contiguous chunks whose
 *              partials (fp32 output + log-sum-exp) are merged by the combine
 *              kernel on the same stream.  -128..-2 = split only the rows of
 *              decode sequences (q_len * Hq / Hkv <= 32) that many ways and
 *              combine only those rows; the other rows are computed unsplit
 *              (-1 = no split).  Automatic choice does this for a batch with
 *              prefill work that stays unsplit and may hold decode sequences
 *              (T - (S - 1) * max_seqlen_q <= 32 / (Hq / Hkv)): one split per
 *              4096 keys of max_seqlen_k, at most 8.
 * workspace,   device scratch for the partials, at least
 * workspace_bytes  ua_workspace_size(T, Hq, D, splits) bytes, 256-byte
 *              aligned; may be NULL when no split is used.  Automatic split
 *              choice (num_splits = 0) never picks a split the workspace
 *              cannot hold.
 * lse_out      optional [T, Hq] fp32 natural-log log-sum-exp of each row's
 *              scaled scores (NULL = not written).
 * test_barrier_timeout  0, or 1 as a test hook only.  Split launches with
 *              prefill work run two 4-wave key groups per workgroup that
 *              synchronise through a polled LDS counter; each wait gives up
 *              after a bounded number of polls (2^20), and a workgroup in
 *              which any wait gave up writes NaN to its rows (output and
 *              log-sum-exp) instead of a result.  1 makes every such wait
 *              give up at once, so a test can see that no timed-out wait
 *              passes silently; every kernel still runs to its end.
 *
 * Requirements checked on the host: abi_version == UA_ABI_VERSION; non-NULL
 * q, k_cache, v_cache, out, cu_seqlens_q, seqused_k, block_table (when S > 0
 * and T > 0); D == 128; Hq % Hkv == 0 and Hq / Hkv <= 128; bs a power of two
 * in [16, 4096]; W >= ceil(max_seqlen_k / bs); all strides multiples of 8 and
 * positive, kv_stride_slot < 2^26; q, out, k_cache, v_cache 16-byte aligned;
 * -128 <= num_splits <= 128.
 * S == 0 or T == 0 is a no-op that returns UA_OK.
 */
typedef struct ua_attn_params {
    uint32_t abi_version;
    int32_t q_dtype;                 /* ua_dtype of q and out */
    int32_t kv_dtype;                /* ua_dtype of k_cache and v_cache */
    int32_t causal;

    const void *q;
    const void *k_cache;
    const void *v_cache;
    void *out;
    const int32_t *cu_seqlens_q;
    const int32_t *seqused_k;
    const int32_t *block_table;
    const float *k_scale;
    const float *v_scale;
    float *lse_out;
    void *workspace;
    uint64_t workspace_bytes;

    int64_t q_stride_token, q_stride_head;
    int64_t o_stride_token, o_stride_head;
    int64_t kv_stride_block, kv_stride_slot, kv_stride_head;

    int32_t num_seqs, num_tokens, num_q_heads, num_kv_heads;
    int32_t head_size, block_size, num_blocks, block_table_stride;
    int32_t max_seqlen_q, max_seqlen_k;
    int32_t num_splits;
    float softmax_scale;
    int32_t window_left;             /* -1 = unbounded */
    int32_t window_right;            /* -1 = unbounded */
    const float *alibi_slopes;       /* [Hq] or NULL */
    int32_t fp8_compute;             /* 0 or 1 */
    int32_t test_barrier_timeout;    /* 0 (1: test hook, see above) */
} ua_attn_params;

/* The launch the library chose for a call (filled by ua_plan).  Two kernels
 * share the work: the prefill kernel (4 waves x 32 query rows of one kv head
 * share each 64-key tile) and the decode kernel (every sequence with
 * q_len * (Hq / Hkv) <= 32 query rows: 4 waves stream disjoint 32-key units
 * and merge).  When max_seqlen_q * (Hq / Hkv) <= 32 only the decode kernel
 * runs.  Otherwise the prefill kernel runs, and the decode kernel runs beside
 * it (the prefill kernel then skipping the short sequences) only when some
 * sequence can be short: when num_tokens - (num_seqs - 1) * max_seqlen_q
 * <= 32 / (Hq / Hkv).
 * Split launches with prefill work use 8-wave workgroups: two groups of 4
 * prefill waves take alternate tiles of the split and merge, and the decode
 * body streams with 8 waves; when such a launch has at most 8 x 256
 * workgroups' worth of items ((grid_x + decode_grid_x) x grid_y), it runs as
 * min(items, 256) workgroups, workgroup w taking items w, w + 256, ... in
 * grid order.  A launch that splits only the decode rows
 * (kernels bit 2) keeps 4-wave workgroups: decode_grid_x decode workgroups
 * (sequence x kv head x split) spread among the grid_x prefill workgroups in
 * one dimension, grid_y = 1. */
typedef struct ua_plan_info {
    int32_t block_m;       /* query rows per prefill workgroup */
    int32_t block_q;       /* query tokens per prefill workgroup = block_m / (Hq / Hkv) */
    int32_t tile_n;        /* keys per prefill KV tile */
    int32_t num_waves;     /* 64-lane wavefronts per workgroup (both bodies): 4, or 8 for split
                              launches with prefill work (two key groups per query block) */
    int32_t num_splits;    /* splits actually used (1 = no combine launch) */
    int32_t kernels;       /* bit 0: prefill kernel launched; bit 1: decode kernel launched;
                              bit 2: only the decode rows are split (num_splits ways) */
    int64_t grid_x;        /* prefill workgroups along (query block slot x kv head); 0 if not launched */
    int64_t grid_y;        /* workgroups along splits (both kernels); 1 when bit 2 is set */
    int64_t decode_grid_x; /* decode workgroups along (sequence x kv head), times num_splits
                              when bit 2 is set; 0 if not launched */
} ua_plan_info;

/*
 * Attention forward (the unified paged varlen path).  Enqueues the attention
 * kernel and, when more than one split is used, the combine kernel, on
 * `stream`.  Returns UA_OK once enqueued; see ua_status for errors.
 */
ua_status ua_unified_attention(const ua_attn_params *p, void *stream);

/*
 * Log-sum-exp merge of split partials (page "flashatten takeaways EP2 工程",
 * section "源代码接口"): for each row r (token, q head),
 *   L = max_p lse[p, r];  w_p = exp(lse[p, r] - L);
 *   out[r] = sum_p w_p * o[p, r] / sum_p w_p;  lse_out[r] = L + ln sum_p w_p.
 * Splits with lse = -inf weigh 0; a row whose splits are all -inf gets out = 0
 * and lse_out = -inf.
 * o_partial    [num_splits, T, Hq, D] fp32, contiguous (normalised partials).
 * lse_partial  [num_splits, T, Hq] fp32, contiguous, natural log.
 * out          [T, Hq, D] of out_dtype (bf16 or fp16), strides o_stride_*.
 * lse_out      optional [T, Hq] fp32 (NULL = not written).
 * Requirements: 1 <= num_splits <= 128, D == 128, non-NULL o_partial,
 * lse_partial, out; 16-byte aligned pointers; strides multiples of 8.
 */
ua_status ua_split_kv_combine(const float *o_partial, const float *lse_partial,
                              int32_t num_splits, int32_t num_tokens, int32_t num_q_heads,
                              int32_t head_size, void *out, int32_t out_dtype,
                              int64_t o_stride_token, int64_t o_stride_head,
                              float *lse_out, void *stream);

/* Bytes of workspace a split call needs: o_partial (fp32 [P, T, Hq, D],
 * rounded up to 256 bytes) followed by lse_partial (fp32 [P, T, Hq]).
 * Returns 0 when num_splits <= 1. */
size_t ua_workspace_size(int32_t num_tokens, int32_t num_q_heads, int32_t head_size,
                         int32_t num_splits);

/*
 * ua_unified_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The same computation and kernels, with the split partials in
 * the library's own scratch array instead of a caller workspace: one array of
 * UA_NOALLOC_SCRATCH_BYTES per GPU the library runs on, held until the
 * process ends.  p->workspace and p->workspace_bytes are ignored; automatic
 * splits (num_splits = 0) are chosen within the scratch.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first
 * split call on a device looks up that device's array address.
 *
 * Errors: as ua_unified_attention, plus UA_ERR_SCRATCH when the requested
 * splits need more than UA_NOALLOC_SCRATCH_BYTES
 * (ua_workspace_size(T, Hq, D, splits) > UA_NOALLOC_SCRATCH_BYTES); nothing
 * is enqueued then.
 *
 * Calls that overlap on one GPU (on different streams, or from different
 * threads without ordering) share its array and race: order them.  The array
 * keeps the last call's partials; nothing in it needs to start at zero.
 */
#define UA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ua_status ua_unified_attention_noalloc(const ua_attn_params *p, void *stream);

/* The launch ua_unified_attention would make for *p (host only, no HIP call).
 * Validates *p exactly as ua_unified_attention does. */
ua_status ua_plan(const ua_attn_params *p, ua_plan_info *plan);

/*
 * KV-cache append (page "flashatten takeaways EP2 工程", section "kv cache":
 * the cache of a sequence grows by the new tokens' k and v rows; section
 * "源代码接口": the split-KV launch's Append_KV switch).  Writes the k and v
 * rows of the new tokens into their page slots, converted to the cache dtype:
 * token i of sequence s (packed row cu_seqlens_q[s] + i, i < q_len(s)) sits
 * at key position kv_len(s) - q_len(s) + i (the newest positions, as in the
 * causal convention of ua_attn_params), i.e. in physical block
 * block_table[s * W + pos / bs], slot pos % bs.
 *
 * k_new,       [T, Hkv, D] of new_dtype (bf16 or fp16); strides
 * v_new        new_stride_token, new_stride_head (elements).
 * k_cache,     [NB, bs, Hkv, D] of cache_dtype (new_dtype, or fp8 e4m3fn);
 * v_cache      strides kv_stride_block, kv_stride_slot, kv_stride_head.
 *              Only the appended rows are written.
 * cu_seqlens_q [S + 1] int32 as in ua_attn_params (new tokens per sequence).
 * seqused_k    [S] int32: kv_len(s) AFTER the append (>= q_len(s)).
 * block_table  [S, W] int32; the pages holding the new positions must be
 *              allocated by the caller.
 * k_scale,     device fp32 scalars, required iff cache_dtype is fp8 (else
 * v_scale      NULL): a value x is stored as the e4m3fn code nearest to
 *              x / scale (round to nearest, ties to even), saturated to +-448.
 *
 * Requirements checked on the host: abi_version == UA_ABI_VERSION; non-NULL
 * k_new, v_new, k_cache, v_cache, cu_seqlens_q, seqused_k, block_table (when
 * S > 0 and T > 0); D == 128; bs a power of two in [16, 4096]; strides
 * multiples of 8 and positive; 16-byte aligned data pointers; 4-byte aligned
 * k_scale and v_scale.  Rows of tokens that belong to no sequence are not read.  S == 0 or T == 0 is a no-op.
 * Data-dependent violations (positions past the table, block ids outside
 * [0, NB), overlapping sequences) are undefined behaviour.
 */
typedef struct ua_append_params {
    uint32_t abi_version;
    int32_t new_dtype;               /* ua_dtype of k_new and v_new */
    int32_t cache_dtype;             /* ua_dtype of k_cache and v_cache */
    int32_t reserved;

    const void *k_new;
    const void *v_new;
    void *k_cache;
    void *v_cache;
    const int32_t *cu_seqlens_q;
    const int32_t *seqused_k;
    const int32_t *block_table;
    const float *k_scale;
    const float *v_scale;

    int64_t new_stride_token, new_stride_head;
    int64_t kv_stride_block, kv_stride_slot, kv_stride_head;

    int32_t num_seqs, num_tokens, num_kv_heads, head_size;
    int32_t block_size, num_blocks, block_table_stride;
    int32_t reserved2;
} ua_append_params;

/* Enqueue the append kernel on `stream`.  Returns UA_OK once enqueued. */
ua_status ua_kv_append(const ua_append_params *p, void *stream);

/* sizeof(ua_append_params) of the built library. */
size_t ua_append_params_size(void);

/*
 * Attention backward (page "Fused Attention", the tutorial's backward pass:
 * the preprocess forming Delta = rowsum(O * dO), the dK/dV loop and the dQ
 * loop, both recomputing the weights P from the forward's log-sum-exp).  For
 * the loss sum(dO * O) of O = softmax(scale * Q K^T) V under the forward's
 * mask, writes
 *     dQ = scale * dS K,   dK = scale * dS^T Q,   dV = P^T dO,
 *     dS = P * (dO V^T - Delta),
 * where a kv head's dK and dV sum the contributions of the Hq / Hkv query
 * heads that read it (query head h reads kv head h / (Hq / Hkv)).  Training
 * has no cache: k and v are dense, packed like the queries.
 *
 * q, out, dout [T, Hq, 128] bf16 or fp16 (dtype), contiguous: sequence s owns
 *              rows cu_seqlens_q[s] .. cu_seqlens_q[s+1] - 1.
 * k, v         [Tk, Hkv, 128] of dtype, contiguous: sequence s owns rows
 *              cu_seqlens_k[s] .. cu_seqlens_k[s+1] - 1 (kv_len(s) keys).
 * lse          [T, Hq] fp32, natural-log log-sum-exp of each row as the
 *              forward writes it (ua_attn_params.lse_out); -inf for a row
 *              that sees no key (its gradients are 0).
 * dq           [T, Hq, 128], dk, dv [Tk, Hkv, 128] of dtype, written in full
 *              (keys no query sees get dK = dV = 0).
 * causal       bottom-right alignment as in the forward: query i of a
 *              sequence sits at key position kv_len - q_len + i.
 * workspace    device memory of at least ua_bwd_workspace_size(T, Hq)
 *              bytes, 256-byte aligned, no contents kept between calls.
 *
 * Requirements checked on the host: abi_version == UA_ABI_VERSION; dtype bf16
 * or fp16; head_size == 128; Hq a multiple of Hkv with Hq / Hkv <= 128;
 * non-NULL, 16-byte aligned tensors when T > 0; T * Hq and Tk * Hkv below
 * 2^23 (UA_ERR_UNSUPPORTED beyond).  S == 0 or T + Tk == 0 is a no-op.
 * Data-dependent violations (cu_seqlens not non-decreasing or not ending at
 * T / Tk) are undefined behaviour.  Overlapping output and input tensors race.
 */
typedef struct ua_bwd_params {
    uint32_t abi_version;
    int32_t dtype;                   /* ua_dtype of q, k, v, out, dout, dq, dk, dv */
    int32_t causal;
    float softmax_scale;

    const void *q;
    const void *k;
    const void *v;
    const void *out;
    const void *dout;
    const float *lse;
    const int32_t *cu_seqlens_q;
    const int32_t *cu_seqlens_k;
    void *dq;
    void *dk;
    void *dv;
    void *workspace;
    uint64_t workspace_bytes;

    int32_t num_seqs, num_tokens, num_tokens_k, num_q_heads, num_kv_heads, head_size;
} ua_bwd_params;

/* Enqueue the backward kernels on `stream`.  Returns UA_OK once enqueued. */
ua_status ua_attention_backward(const ua_bwd_params *p, void *stream);

/* Workspace bytes ua_attention_backward needs: two fp32 values per (token,
 * query head) row (LSE in log2 units and Delta), rounded up. */
size_t ua_bwd_workspace_size(int32_t num_tokens, int32_t num_q_heads);

/* sizeof(ua_bwd_params) of the built library. */
size_t ua_bwd_params_size(void);

/* Static text for a status code. */
const char *ua_status_string(int32_t status);

/* UA_ABI_VERSION of the built library. */
uint32_t ua_abi_version(void);

/* Fill *p with the defaults: every field zero / NULL except abi_version =
 * UA_ABI_VERSION, window_left = window_right = -1 (no local window) and
 * num_splits = 1.  The caller then sets the tensors, shapes, strides and
 * softmax_scale.  No-op for p == NULL. */
void ua_attn_params_init(ua_attn_params *p);

/* sizeof(ua_attn_params) and sizeof(ua_plan_info) of the built library, so a
 * binding can check its mirror of the structs. */
size_t ua_params_size(void);
size_t ua_plan_info_size(void);

#ifdef __cplusplus
}
#endif

#endif /* UA_H */
