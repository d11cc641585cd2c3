// C-ABI layer: argument validation, launch planning and kernel enqueue.
//
// The host side of the unified attention call (page "vLLM Triton unified
// attention notes", section unified_attention: assertions, shape parameters,
// num_queries_per_kv and the query-block count are derived on the host, and
// the grid is sized there without reading device memory).  The split path
// mirrors the two-step interface of page "flashatten takeaways EP2 工程",
// section "源代码接口": the partial pass, then the combine on the same stream,
// at most 128 splits.

#include "ua.h"
#include "ua_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

namespace {

constexpr int kMaxSplits = 128;
constexpr int kMaxGroup = 128;
constexpr size_t kAlign = 256;
constexpr int kNumCUs = 256;
constexpr int kBarrierPolls = 1 << 20;   // polls before a key-group barrier wait gives up
// Automatic split of a mixed batch's decode rows: one split per this many keys
// of the longest sequence, at most kMaxDecodeSplits.
constexpr int kDecodeSplitKeys = 4096;
constexpr int kMaxDecodeSplits = 8;
// Split launches with prefill work (whole-CU workgroups) of at most this many
// items per CU run as one persistent workgroup per CU.
constexpr int kPersistItemsPerCU = 8;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int64_t x) {
    int r = 0;
    while ((int64_t(1) << r) < x)
        ++r;
    return r;
}
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t partial_o_bytes(int64_t T, int64_t Hq, int64_t D, int64_t P) {
    return round_up((size_t)(P * T * Hq * D) * sizeof(float), kAlign);
}

// Checks of ua_attn_params that need no device access.  The order fixes which
// status a call with several faults gets: ABI, sizes, dtypes, shapes,
// pointers, strides, splits, workspace.
ua_status validate(const ua_attn_params *p) {
    if (p == nullptr || p->abi_version != UA_ABI_VERSION)
        return UA_ERR_INVALID_ARG;
    if (p->num_seqs < 0 || p->num_tokens < 0)
        return UA_ERR_INVALID_ARG;
    if (p->num_splits < -kMaxSplits || p->num_splits > kMaxSplits)
        return UA_ERR_INVALID_ARG;
    if (p->num_seqs == 0 || p->num_tokens == 0)
        return UA_OK;                                          // nothing to do
    if (p->q_dtype != UA_BF16 && p->q_dtype != UA_FP16)
        return p->q_dtype == UA_FP8_E4M3FN ? UA_ERR_UNSUPPORTED : UA_ERR_INVALID_ARG;
    if (p->kv_dtype != UA_BF16 && p->kv_dtype != UA_FP16 && p->kv_dtype != UA_FP8_E4M3FN)
        return UA_ERR_INVALID_ARG;
    if (p->kv_dtype != p->q_dtype && p->kv_dtype != UA_FP8_E4M3FN)
        return UA_ERR_UNSUPPORTED;                             // e.g. bf16 q with fp16 cache
    if (p->head_size <= 0 || p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->block_size <= 0 ||
        p->num_blocks <= 0 || p->block_table_stride <= 0 || p->max_seqlen_q < 0 || p->max_seqlen_k < 0)
        return UA_ERR_INVALID_ARG;
    if (p->head_size != ua::kHeadSize)
        return UA_ERR_UNSUPPORTED;
    if (p->num_q_heads % p->num_kv_heads != 0)
        return UA_ERR_INVALID_ARG;
    if (p->num_q_heads / p->num_kv_heads > kMaxGroup)
        return UA_ERR_UNSUPPORTED;
    if (!pow2(p->block_size) || p->block_size < 16 || p->block_size > 4096)
        return UA_ERR_UNSUPPORTED;
    if ((int64_t)p->block_table_stride * p->block_size < p->max_seqlen_k)
        return UA_ERR_INVALID_ARG;                             // table too narrow for max_seqlen_k
    if (!(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.0f))
        return UA_ERR_INVALID_ARG;
    if (p->causal != 0 && p->causal != 1)
        return UA_ERR_INVALID_ARG;
    if (p->window_left < -1 || p->window_right < -1 || !aligned(p->alibi_slopes, 4))
        return UA_ERR_INVALID_ARG;
    if (p->alibi_slopes && p->max_seqlen_k > (1 << 24))
        return UA_ERR_UNSUPPORTED;                             // positions exact in fp32
    if ((p->fp8_compute != 0 && p->fp8_compute != 1) ||
        (p->test_barrier_timeout != 0 && p->test_barrier_timeout != 1))
        return UA_ERR_INVALID_ARG;
    if (p->fp8_compute && (p->kv_dtype != UA_FP8_E4M3FN || p->window_left >= 0 ||
                           p->window_right >= 0 || p->alibi_slopes))
        return UA_ERR_UNSUPPORTED;
    if (!p->q || !p->k_cache || !p->v_cache || !p->out || !p->cu_seqlens_q || !p->seqused_k ||
        !p->block_table)
        return UA_ERR_INVALID_ARG;
    if (!aligned(p->q, 16) || !aligned(p->k_cache, 16) || !aligned(p->v_cache, 16) ||
        !aligned(p->out, 16) || !aligned(p->cu_seqlens_q, 4) || !aligned(p->seqused_k, 4) ||
        !aligned(p->block_table, 4) || !aligned(p->lse_out, 4))
        return UA_ERR_INVALID_ARG;
    if (p->kv_dtype == UA_FP8_E4M3FN &&
        (!p->k_scale || !p->v_scale || !aligned(p->k_scale, 4) || !aligned(p->v_scale, 4)))
        return UA_ERR_INVALID_ARG;
    const int64_t strides[] = {p->q_stride_token, p->q_stride_head, p->o_stride_token,
                               p->o_stride_head, p->kv_stride_block, p->kv_stride_slot,
                               p->kv_stride_head};
    for (int64_t st : strides)
        if (st <= 0 || st % 8 != 0)
            return UA_ERR_INVALID_ARG;
    if (p->kv_stride_slot >= (int64_t(1) << 26))
        return UA_ERR_UNSUPPORTED;                             // per-lane 32-bit page offsets
    return UA_OK;
}

struct Plan {
    bool prefill;          // launch the prefill kernel
    bool decode;           // launch the decode kernel
    int32_t block_q;       // tokens per prefill workgroup
    int32_t splits;
    int64_t qslots;        // prefill query-block slots
    bool wide;             // 8-wave workgroups: two prefill key groups per query block
    bool mix;              // only the decode rows are split (prefill rows unsplit)
};

// Whether some sequence can be a decode sequence (q_len * G <= kDecodeRows)
// given only T, S and max_seqlen_q: the shortest sequence has at least
// T - (S - 1) * max_seqlen_q tokens.
bool may_have_decode_rows(const ua_attn_params *p, int G) {
    return (int64_t)p->num_tokens - (int64_t)(p->num_seqs - 1) * p->max_seqlen_q <=
           ua::kDecodeRows / G;
}

// Kernel choice: every sequence with q_len * G <= kDecodeRows rows goes to the
// decode kernel; when max_seqlen_q * G <= kDecodeRows that is every sequence
// and the prefill kernel is not launched.  Split choice for num_splits = 0,
// within what the workspace holds and keeping at least 8 prefill tiles / 8
// decode units per split: launches with prefill work aim at about two rounds
// of workgroups over the CUs (two 4-wave workgroups per CU); decode-only
// launches at about eight rounds, since their workgroups are short and
// memory-bound and more of them balance uneven key lengths (on the 256 x
// (1 query, 512..8192 keys) decode batch 2 splits stream best, 8 cost ~6%).
// A launch with prefill work that stays unsplit and may hold decode sequences
// splits only the decode rows, one split per kDecodeSplitKeys keys of the
// longest sequence (at most kMaxDecodeSplits): its decode workgroups are then
// short and are spread among the prefill ones instead of occupying every slot
// at the start.  num_splits = -n asks for that decode-only split explicitly.
Plan make_plan(const ua_attn_params *p) {
    Plan pl;
    const int G = p->num_q_heads / p->num_kv_heads;
    const bool decode_only = (int64_t)p->max_seqlen_q * G <= ua::kDecodeRows;
    pl.prefill = !decode_only;
    // the decode kernel runs only where some sequence can be a decode
    // sequence (its workgroups would otherwise all exit at once)
    pl.decode = decode_only || may_have_decode_rows(p, G);
    pl.block_q = ua::kPrefillBlockM / G;
    pl.qslots = (int64_t)p->num_tokens / pl.block_q + p->num_seqs;
    pl.mix = false;
    int splits = p->num_splits;
    if (splits < 0) {
        splits = -splits;
        pl.mix = pl.prefill;            // decode-only launches: every row is a decode row
        if (pl.prefill && !pl.decode)
            splits = 1;                 // no decode rows to split
    }
    if (splits == 0) {
        int64_t units;
        int64_t min_keys;
        if (decode_only) {
            units = (int64_t)p->num_seqs * p->num_kv_heads;
            min_keys = 8 * ua::kDecodeUnit;
        } else {
            const int64_t blocks_per_seq = ((int64_t)p->max_seqlen_q + pl.block_q - 1) / pl.block_q;
            units = std::min<int64_t>(pl.qslots, p->num_seqs * std::max<int64_t>(blocks_per_seq, 1)) *
                    p->num_kv_heads;
            min_keys = 8 * ua::kPrefillTileN;
        }
        const int64_t wg_wanted = (decode_only ? 8LL : 2LL) * kNumCUs * 2;
        int64_t want = units > 0 ? (wg_wanted + units - 1) / units : 1;
        const int64_t max_by_len = std::max<int64_t>(1, p->max_seqlen_k / min_keys);
        want = std::min<int64_t>({want, max_by_len, (int64_t)kMaxSplits});
        splits = (int)std::max<int64_t>(1, want);
        while (splits > 1 && ua_workspace_size(p->num_tokens, p->num_q_heads, p->head_size, splits) >
                                 (p->workspace ? p->workspace_bytes : 0))
            --splits;
        if (!decode_only && splits <= 1 && may_have_decode_rows(p, G)) {
            int ds = (int)std::min<int64_t>(kMaxDecodeSplits, p->max_seqlen_k / kDecodeSplitKeys);
            while (ds > 1 && ua_workspace_size(p->num_tokens, p->num_q_heads, p->head_size, ds) >
                                 (p->workspace ? p->workspace_bytes : 0))
                --ds;
            if (ds > 1) {
                splits = ds;
                pl.mix = true;
            }
        }
    }
    pl.splits = std::max(1, splits);
    if (pl.splits == 1)
        pl.mix = false;
    // A split launch with prefill work has few query blocks per kv head (that
    // is why it splits): its prefill workgroups run two key groups over
    // alternate tiles, so that one workgroup per CU still puts two waves on
    // every SIMD.
    pl.wide = pl.prefill && pl.splits > 1 && !pl.mix;
    return pl;
}

// Host-checkable requirements of ua_kv_append (see ua.h).
ua_status validate_append(const ua_append_params *p) {
    if (p == nullptr || p->abi_version != UA_ABI_VERSION)
        return UA_ERR_INVALID_ARG;
    if (p->num_seqs < 0 || p->num_tokens < 0 || p->num_kv_heads <= 0 || p->num_blocks < 0 ||
        p->block_table_stride < 0)
        return UA_ERR_INVALID_ARG;
    if (p->new_dtype != UA_BF16 && p->new_dtype != UA_FP16)
        return p->new_dtype == UA_FP8_E4M3FN ? UA_ERR_UNSUPPORTED : UA_ERR_INVALID_ARG;
    if (p->cache_dtype != p->new_dtype && p->cache_dtype != UA_FP8_E4M3FN)
        return (p->cache_dtype == UA_BF16 || p->cache_dtype == UA_FP16) ? UA_ERR_UNSUPPORTED
                                                                        : UA_ERR_INVALID_ARG;
    if (p->head_size != ua::kHeadSize)
        return UA_ERR_UNSUPPORTED;
    if (!pow2(p->block_size) || p->block_size < 16 || p->block_size > 4096)
        return UA_ERR_INVALID_ARG;
    if (p->num_seqs == 0 || p->num_tokens == 0)
        return UA_OK;
    if (!p->k_new || !p->v_new || !p->k_cache || !p->v_cache || !p->cu_seqlens_q || !p->seqused_k ||
        !p->block_table)
        return UA_ERR_INVALID_ARG;
    const bool fp8 = p->cache_dtype == UA_FP8_E4M3FN;
    if (fp8 && (!p->k_scale || !p->v_scale || !aligned(p->k_scale, 4) || !aligned(p->v_scale, 4)))
        return UA_ERR_INVALID_ARG;
    const int64_t strides[] = {p->new_stride_token, p->new_stride_head, p->kv_stride_block,
                               p->kv_stride_slot, p->kv_stride_head};
    for (int64_t st : strides)
        if (st <= 0 || st % 8 != 0)
            return UA_ERR_INVALID_ARG;
    if (!aligned(p->k_new, 16) || !aligned(p->v_new, 16) || !aligned(p->k_cache, 16) ||
        !aligned(p->v_cache, 16))
        return UA_ERR_INVALID_ARG;
    if ((int64_t)p->num_tokens * p->num_kv_heads > (int64_t)0x7fffffff * 16)
        return UA_ERR_UNSUPPORTED;
    return UA_OK;
}

// backward workspace: [Hq][T] LSE2 then [Hq][T] Delta, each padded by 64 floats
size_t bwd_half_bytes(int64_t T, int64_t Hq) { return round_up((size_t)(Hq * T + 64) * sizeof(float), kAlign); }

ua_status validate_bwd(const ua_bwd_params *p) {
    if (p == nullptr || p->abi_version != UA_ABI_VERSION)
        return UA_ERR_INVALID_ARG;
    if (p->dtype != UA_BF16 && p->dtype != UA_FP16)
        return p->dtype == UA_FP8_E4M3FN ? UA_ERR_UNSUPPORTED : UA_ERR_INVALID_ARG;
    if (p->causal != 0 && p->causal != 1)
        return UA_ERR_INVALID_ARG;
    if (p->num_seqs < 0 || p->num_tokens < 0 || p->num_tokens_k < 0 || p->num_q_heads <= 0 ||
        p->num_kv_heads <= 0 || p->num_q_heads % p->num_kv_heads != 0)
        return UA_ERR_INVALID_ARG;
    if (p->head_size != ua::kHeadSize || p->num_q_heads / p->num_kv_heads > kMaxGroup)
        return UA_ERR_UNSUPPORTED;
    if (!(std::isfinite(p->softmax_scale)))
        return UA_ERR_INVALID_ARG;
    if (p->num_seqs == 0 || (p->num_tokens == 0 && p->num_tokens_k == 0))
        return UA_OK;
    if (!p->cu_seqlens_q || !p->cu_seqlens_k)
        return UA_ERR_INVALID_ARG;
    const void *tensors[] = {p->q, p->out, p->dout, p->dq, p->k, p->v, p->dk, p->dv};
    const bool present[] = {p->num_tokens > 0, p->num_tokens > 0, p->num_tokens > 0, p->num_tokens > 0,
                            p->num_tokens_k > 0, p->num_tokens_k > 0, p->num_tokens_k > 0,
                            p->num_tokens_k > 0};
    for (int i = 0; i < 8; ++i)
        if (present[i] && (tensors[i] == nullptr || !aligned(tensors[i], 16)))
            return UA_ERR_INVALID_ARG;
    if (p->num_tokens > 0 && (p->lse == nullptr || !aligned(p->lse, 4)))
        return UA_ERR_INVALID_ARG;
    // 32-bit per-lane row offsets inside the kernels
    if ((int64_t)p->num_tokens * p->num_q_heads >= (int64_t(1) << 23) ||
        (int64_t)p->num_tokens_k * p->num_kv_heads >= (int64_t(1) << 23))
        return UA_ERR_UNSUPPORTED;
    if (p->num_tokens > 0 &&
        (p->workspace == nullptr || !aligned(p->workspace, kAlign) ||
         p->workspace_bytes < 2 * bwd_half_bytes(p->num_tokens, p->num_q_heads)))
        return UA_ERR_WORKSPACE;
    return UA_OK;
}

}  // namespace

extern "C" {

uint32_t ua_abi_version(void) { return UA_ABI_VERSION; }

void ua_attn_params_init(ua_attn_params *p) {
    if (p == nullptr)
        return;
    std::memset(p, 0, sizeof(*p));
    p->abi_version = UA_ABI_VERSION;
    p->window_left = -1;
    p->window_right = -1;
    p->num_splits = 1;
}
size_t ua_params_size(void) { return sizeof(ua_attn_params); }
size_t ua_plan_info_size(void) { return sizeof(ua_plan_info); }
size_t ua_append_params_size(void) { return sizeof(ua_append_params); }

ua_status ua_kv_append(const ua_append_params *p, void *stream) {
    const ua_status st = validate_append(p);
    if (st != UA_OK)
        return st;
    if (p->num_seqs == 0 || p->num_tokens == 0)
        return UA_OK;
    ua::AppendArgs a{};
    a.k_new = p->k_new;
    a.v_new = p->v_new;
    a.k_cache = p->k_cache;
    a.v_cache = p->v_cache;
    a.cu_seqlens_q = p->cu_seqlens_q;
    a.seqused_k = p->seqused_k;
    a.block_table = p->block_table;
    a.k_scale = p->cache_dtype == UA_FP8_E4M3FN ? p->k_scale : nullptr;
    a.v_scale = p->cache_dtype == UA_FP8_E4M3FN ? p->v_scale : nullptr;
    a.new_st_tok = p->new_stride_token;
    a.new_st_head = p->new_stride_head;
    a.kv_st_blk = p->kv_stride_block;
    a.kv_st_slot = p->kv_stride_slot;
    a.kv_st_head = p->kv_stride_head;
    a.bt_stride = p->block_table_stride;
    a.num_seqs = p->num_seqs;
    a.num_tokens = p->num_tokens;
    a.num_kv_heads = p->num_kv_heads;
    a.log2_block_size = ilog2(p->block_size);
    if (ua::launch_append(a, p->new_dtype == UA_FP16, p->cache_dtype == UA_FP8_E4M3FN,
                          static_cast<hipStream_t>(stream)) != hipSuccess)
        return UA_ERR_HIP;
    return UA_OK;
}

size_t ua_bwd_params_size(void) { return sizeof(ua_bwd_params); }

size_t ua_bwd_workspace_size(int32_t num_tokens, int32_t num_q_heads) {
    if (num_tokens <= 0 || num_q_heads <= 0)
        return 0;
    return 2 * bwd_half_bytes(num_tokens, num_q_heads);
}

ua_status ua_attention_backward(const ua_bwd_params *p, void *stream) {
    const ua_status st = validate_bwd(p);
    if (st != UA_OK)
        return st;
    if (p->num_seqs == 0 || (p->num_tokens == 0 && p->num_tokens_k == 0))
        return UA_OK;
    ua::BwdArgs a{};
    a.q = p->q;
    a.k = p->k;
    a.v = p->v;
    a.o = p->out;
    a.dout = p->dout;
    a.lse = p->lse;
    a.cu_seqlens_q = p->cu_seqlens_q;
    a.cu_seqlens_k = p->cu_seqlens_k;
    a.dq = p->dq;
    a.dk = p->dk;
    a.dv = p->dv;
    a.num_seqs = p->num_seqs;
    a.num_tokens = p->num_tokens;
    a.num_tokens_k = p->num_tokens_k;
    a.num_q_heads = p->num_q_heads;
    a.num_kv_heads = p->num_kv_heads;
    a.group = p->num_q_heads / p->num_kv_heads;
    a.block_q = ua::kPrefillBlockM / a.group;
    a.q_slots = p->num_tokens / a.block_q + p->num_seqs;
    a.dkdv_wgs = (p->num_tokens_k / 128 + p->num_seqs) * p->num_kv_heads;
    a.dq_wgs = p->num_tokens > 0 ? a.q_slots * p->num_kv_heads : 0;
    a.scale = p->softmax_scale;
    uint8_t *ws = static_cast<uint8_t *>(p->workspace);
    a.lse2 = reinterpret_cast<float *>(ws);
    a.delta = reinterpret_cast<float *>(ws + (ws ? bwd_half_bytes(p->num_tokens, p->num_q_heads) : 0));
    if (ua::launch_backward(a, p->dtype == UA_FP16, p->causal != 0, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return UA_ERR_HIP;
    return UA_OK;
}

const char *ua_status_string(int32_t status) {
    switch (status) {
    case UA_OK: return "ok";
    case UA_ERR_INVALID_ARG: return "invalid argument";
    case UA_ERR_UNSUPPORTED: return "unsupported configuration";
    case UA_ERR_WORKSPACE: return "workspace missing or too small for the requested splits";
    case UA_ERR_HIP: return "HIP runtime error";
    case UA_ERR_SCRATCH:
        return "the requested splits need more than the no-allocation scratch (UA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

size_t ua_workspace_size(int32_t num_tokens, int32_t num_q_heads, int32_t head_size,
                         int32_t num_splits) {
    if (num_splits <= 1 || num_tokens <= 0 || num_q_heads <= 0 || head_size <= 0)
        return 0;
    return partial_o_bytes(num_tokens, num_q_heads, head_size, num_splits) +
           round_up((size_t)num_splits * num_tokens * num_q_heads * sizeof(float), kAlign);
}

ua_status ua_plan(const ua_attn_params *p, ua_plan_info *plan) {
    if (plan == nullptr)
        return UA_ERR_INVALID_ARG;
    std::memset(plan, 0, sizeof(*plan));
    const ua_status st = validate(p);
    if (st != UA_OK)
        return st;
    if (p->num_seqs == 0 || p->num_tokens == 0)
        return UA_OK;
    const Plan pl = make_plan(p);
    if (pl.splits > 1) {
        const size_t need = ua_workspace_size(p->num_tokens, p->num_q_heads, p->head_size, pl.splits);
        if (!p->workspace || !aligned(p->workspace, kAlign) || p->workspace_bytes < need)
            return UA_ERR_WORKSPACE;
    }
    plan->block_m = ua::kPrefillBlockM;
    plan->block_q = pl.block_q;
    plan->tile_n = ua::kPrefillTileN;
    plan->num_waves = pl.wide ? 2 * ua::kWaves : ua::kWaves;
    plan->num_splits = pl.splits;
    plan->kernels = (pl.prefill ? 1 : 0) | (pl.decode ? 2 : 0) | (pl.mix ? 4 : 0);
    plan->grid_x = pl.prefill ? pl.qslots * p->num_kv_heads : 0;
    plan->grid_y = pl.mix ? 1 : pl.splits;
    plan->decode_grid_x =
        pl.decode ? (int64_t)p->num_seqs * p->num_kv_heads * (pl.mix ? pl.splits : 1) : 0;
    return UA_OK;
}

ua_status ua_unified_attention(const ua_attn_params *p, void *stream) {
    ua_plan_info info;
    const ua_status st = ua_plan(p, &info);
    if (st != UA_OK)
        return st;
    if (p->num_seqs == 0 || p->num_tokens == 0)
        return UA_OK;
    if (info.grid_x + info.decode_grid_x > 0x7fffffff - 16)
        return UA_ERR_UNSUPPORTED;
    const Plan pl = make_plan(p);
    const bool split = pl.splits > 1;
    const int G = p->num_q_heads / p->num_kv_heads;

    ua::AttnArgs a{};
    a.q = p->q;
    a.k = p->k_cache;
    a.v = p->v_cache;
    a.out = p->out;
    a.cu_seqlens_q = p->cu_seqlens_q;
    a.seqused_k = p->seqused_k;
    a.block_table = p->block_table;
    a.k_scale = p->kv_dtype == UA_FP8_E4M3FN ? p->k_scale : nullptr;
    a.v_scale = p->kv_dtype == UA_FP8_E4M3FN ? p->v_scale : nullptr;
    a.lse_out = split && !pl.mix ? nullptr : p->lse_out;   // mixed: the prefill rows' own
    if (split) {
        uint8_t *ws = static_cast<uint8_t *>(p->workspace);
        a.o_part = reinterpret_cast<float *>(ws);
        a.lse_part = reinterpret_cast<float *>(
            ws + partial_o_bytes(p->num_tokens, p->num_q_heads, p->head_size, pl.splits));
    }
    a.q_st_tok = p->q_stride_token;
    a.q_st_head = p->q_stride_head;
    a.o_st_tok = p->o_stride_token;
    a.o_st_head = p->o_stride_head;
    a.kv_st_blk = p->kv_stride_block;
    a.kv_st_slot = p->kv_stride_slot;
    a.kv_st_head = p->kv_stride_head;
    a.bt_stride = p->block_table_stride;
    a.num_seqs = p->num_seqs;
    a.num_tokens = p->num_tokens;
    a.num_q_heads = p->num_q_heads;
    a.num_kv_heads = p->num_kv_heads;
    a.group = G;
    a.block_q = pl.block_q;
    a.log2_block_size = ilog2(p->block_size);
    a.num_splits = pl.splits;
    a.num_qslots = (int32_t)pl.qslots;
    a.short_to_decode = pl.decode ? 1 : 0;
    a.scale_log2 = p->softmax_scale * 1.44269504088896341f;

    a.decode_wgs = (int32_t)info.decode_grid_x;
    dim3 grid((unsigned)(info.grid_x + info.decode_grid_x), (unsigned)info.grid_y);
    if (pl.wide && (info.grid_x + info.decode_grid_x) * info.grid_y <= kPersistItemsPerCU * kNumCUs) {
        // whole-CU workgroups, few items: one persistent workgroup per CU
        // walks the items in grid order (see the kernel's persistent loop)
        const int64_t items = (info.grid_x + info.decode_grid_x) * info.grid_y;
        a.persist_items = (int32_t)items;
        a.row_items = (int32_t)(info.grid_x + info.decode_grid_x);
        grid = dim3((unsigned)std::min<int64_t>(items, kNumCUs), 1);
    }
    if (pl.mix) {
        // decode blocks spread over the first half of the grid (see the
        // kernel's MIX entry)
        const int64_t nd = (info.decode_grid_x + 7) / 8, np = (info.grid_x + 7) / 8;
        a.prefill_wgs = (int32_t)info.grid_x;
        a.mix_dblocks = (int32_t)nd;
        a.mix_region = (int32_t)(nd + np / 2);
        grid = dim3((unsigned)(8 * (nd + np)), 1);
    }
    a.win_left = p->window_left;
    a.win_right = p->window_right;
    a.alibi = p->alibi_slopes;
    a.fp8_compute = p->fp8_compute;
    a.spin_limit = p->test_barrier_timeout ? 0 : kBarrierPolls;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool f16 = p->q_dtype == UA_FP16, fp8 = p->kv_dtype == UA_FP8_E4M3FN, causal = p->causal != 0;
    if (ua::launch_attention(a, f16, fp8, causal, split && !pl.mix, pl.wide, pl.mix, grid, s) !=
        hipSuccess)
        return UA_ERR_HIP;
    if (pl.mix) {
        if (ua::launch_combine_decode(a.o_part, a.lse_part, pl.splits,
                                      (int64_t)p->num_tokens * p->num_q_heads, p->num_q_heads,
                                      p->num_kv_heads, p->num_seqs, p->cu_seqlens_q, p->out,
                                      p->q_dtype == UA_FP16, p->o_stride_token, p->o_stride_head,
                                      p->lse_out, s) != hipSuccess)
            return UA_ERR_HIP;
    } else if (split) {
        // rows of tokens past cu_seqlens_q[S] have no partials: the combine
        // leaves them alone, as the unsplit kernel does
        if (ua::launch_combine(a.o_part, a.lse_part, pl.splits,
                               (int64_t)p->num_tokens * p->num_q_heads, p->num_q_heads, p->out,
                               p->q_dtype == UA_FP16, p->o_stride_token, p->o_stride_head,
                               p->lse_out, p->cu_seqlens_q + p->num_seqs, s) != hipSuccess)
            return UA_ERR_HIP;
    }
    return UA_OK;
}

ua_status ua_unified_attention_noalloc(const ua_attn_params *p, void *stream) {
    if (p == nullptr)
        return UA_ERR_INVALID_ARG;
    // validate and plan against the scratch's size before any HIP call (an
    // aligned stand-in address until a split needs the real one)
    ua_attn_params q = *p;
    q.workspace = reinterpret_cast<void *>(kAlign);
    q.workspace_bytes = UA_NOALLOC_SCRATCH_BYTES;
    ua_plan_info info;
    const ua_status st = ua_plan(&q, &info);
    if (st == UA_ERR_WORKSPACE)
        return UA_ERR_SCRATCH;
    if (st != UA_OK)
        return st;
    if (p->num_seqs == 0 || p->num_tokens == 0)
        return UA_OK;
    if (info.num_splits > 1) {
        void *ptr = nullptr;
        if (ua::noalloc_scratch(&ptr) != hipSuccess)
            return UA_ERR_HIP;
        q.workspace = ptr;
        q.num_splits = (info.kernels & 4) ? -info.num_splits : info.num_splits;
    } else {
        q.workspace = nullptr;
        q.workspace_bytes = 0;
        q.num_splits = 1;
    }
    return ua_unified_attention(&q, stream);
}

ua_status ua_split_kv_combine(const float *o_partial, const float *lse_partial, int32_t num_splits,
                              int32_t num_tokens, int32_t num_q_heads, int32_t head_size,
                              void *out, int32_t out_dtype, int64_t o_stride_token,
                              int64_t o_stride_head, float *lse_out, void *stream) {
    if (num_splits < 1 || num_splits > kMaxSplits || num_tokens < 0 || num_q_heads <= 0)
        return UA_ERR_INVALID_ARG;
    if (out_dtype != UA_BF16 && out_dtype != UA_FP16)
        return out_dtype == UA_FP8_E4M3FN ? UA_ERR_UNSUPPORTED : UA_ERR_INVALID_ARG;
    if (head_size <= 0)
        return UA_ERR_INVALID_ARG;
    if (head_size != ua::kHeadSize)
        return UA_ERR_UNSUPPORTED;
    if (num_tokens == 0)
        return UA_OK;
    if (!o_partial || !lse_partial || !out)
        return UA_ERR_INVALID_ARG;
    if (!aligned(o_partial, 16) || !aligned(lse_partial, 4) || !aligned(out, 16) || !aligned(lse_out, 4))
        return UA_ERR_INVALID_ARG;
    if (o_stride_token <= 0 || o_stride_head <= 0 || o_stride_token % 8 || o_stride_head % 8)
        return UA_ERR_INVALID_ARG;
    if (ua::launch_combine(o_partial, lse_partial, num_splits, (int64_t)num_tokens * num_q_heads,
                           num_q_heads, out, out_dtype == UA_FP16, o_stride_token, o_stride_head,
                           lse_out, nullptr, static_cast<hipStream_t>(stream)) != hipSuccess)
        return UA_ERR_HIP;
    return UA_OK;
}

}  // extern "C"
