// Internal interface between the C-ABI layer (ua_api.cpp) and the kernels
// (ua_attention.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ua {

constexpr int kHeadSize = 128;

// Sequences with at most this many query rows (q_len * G) are handled by the
// decode kernel when it is launched.
constexpr int kDecodeRows = 32;

// Arguments of the attention kernels, passed by value.
struct AttnArgs {
    const void *q;
    const void *k;
    const void *v;
    void *out;
    const int32_t *cu_seqlens_q;
    const int32_t *seqused_k;
    const int32_t *block_table;
    const float *k_scale;          // fp8 KV only
    const float *v_scale;
    float *lse_out;                // [T, Hq] or null (unsplit launches only)
    float *o_part;                 // [P, T, Hq, D] (split launches only)
    float *lse_part;               // [P, T, Hq]
    int64_t q_st_tok, q_st_head;
    int64_t o_st_tok, o_st_head;
    int64_t kv_st_blk, kv_st_slot, kv_st_head;
    int64_t bt_stride;
    int32_t num_seqs, num_tokens, num_q_heads, num_kv_heads;
    int32_t group;                 // Hq / Hkv
    int32_t block_q;               // query tokens per prefill workgroup
    int32_t log2_block_size;
    int32_t num_splits;
    int32_t num_qslots;            // T / block_q + S
    int32_t short_to_decode;       // prefill body skips sequences with q_len * G <= kDecodeRows
    int32_t decode_wgs;            // workgroups [0, decode_wgs) run the decode body, the rest prefill
    float scale_log2;              // softmax_scale * log2(e)
    int32_t win_left, win_right;   // local attention bounds (< 0: unbounded)
    const float *alibi;            // [Hq] ALiBi slopes, or null
    int32_t fp8_compute;           // fp8 caches: prefill rows use fp8 MFMA (Q, P rounded to e4m3)
    int32_t spin_limit;            // polls per key-group barrier before it gives up (outputs NaN)
    // mixed launches (prefill rows unsplit, decode rows split num_splits ways):
    int32_t prefill_wgs;           // prefill workgroups (query block slots x kv heads)
    int32_t mix_dblocks;           // blocks of 8 decode workgroups, ceil(decode_wgs / 8)
    int32_t mix_region;            // the decode blocks are spread over grid blocks [0, mix_region)
    // persistent split launches with prefill work (two key groups): items
    // [0, persist_items) in grid order, row_items (decode + prefill
    // workgroups) per split; 0 = one workgroup per item
    int32_t persist_items;
    int32_t row_items;
};

constexpr int kPrefillBlockM = 128;   // query rows per prefill workgroup
constexpr int kPrefillTileN = 64;     // keys per prefill tile
constexpr int kDecodeUnit = 32;       // keys per decode unit
constexpr int kWaves = 4;             // wavefronts per workgroup, both bodies

// Enqueue the attention kernel: grid.x = decode workgroups (S x Hkv) followed
// by prefill workgroups (slots x Hkv), grid.y = splits.  q_f16: q/out are fp16 (else
// bf16); kv_fp8: the cache holds fp8 e4m3fn codes (else the q dtype); wide
// (split launches only): 8-wave workgroups, each prefill workgroup running two
// key groups over alternate tiles of its split.  mix (split = false): only the
// decode rows are split, num_splits ways; decode_wgs = S x Hkv x num_splits,
// prefill_wgs = slots x Hkv, and the one-dimensional grid holds
// 8 x (mix_dblocks + ceil(prefill_wgs / 8)) workgroups.
hipError_t launch_attention(const AttnArgs &a, bool q_f16, bool kv_fp8, bool causal, bool split,
                            bool wide, bool mix, dim3 grid, hipStream_t stream);

// Enqueue the split combine kernel over rows = T * Hq rows.  tok_end:
// optional device pointer to the token count that sequences cover
// (cu_seqlens_q[S]); rows of later tokens are left untouched.
hipError_t launch_combine(const float *o_part, const float *lse_part, int32_t num_splits,
                          int64_t rows, int32_t num_q_heads, void *out, bool out_f16,
                          int64_t o_st_tok, int64_t o_st_head, float *lse_out,
                          const int32_t *tok_end, hipStream_t stream);

// Enqueue the combine of a mixed launch: only the rows of decode sequences
// (q_len * Hq / Hkv <= kDecodeRows) are merged; rows = T * Hq rows per split
// in the partial arrays.
hipError_t launch_combine_decode(const float *o_part, const float *lse_part, int32_t num_splits,
                                 int64_t rows, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t num_seqs, const int32_t *cu_seqlens_q, void *out,
                                 bool out_f16, int64_t o_st_tok, int64_t o_st_head, float *lse_out,
                                 hipStream_t stream);

// Device address of this GPU's no-allocation scratch array
// (UA_NOALLOC_SCRATCH_BYTES bytes, 256-byte aligned), looked up once per device.
hipError_t noalloc_scratch(void **ptr);

// Arguments of the KV-cache append kernel.
struct AppendArgs {
    const void *k_new;
    const void *v_new;
    void *k_cache;
    void *v_cache;
    const int32_t *cu_seqlens_q;
    const int32_t *seqused_k;
    const int32_t *block_table;
    const float *k_scale;          // fp8 cache only
    const float *v_scale;
    int64_t new_st_tok, new_st_head;
    int64_t kv_st_blk, kv_st_slot, kv_st_head;
    int64_t bt_stride;
    int32_t num_seqs, num_tokens, num_kv_heads;
    int32_t log2_block_size;
};

// Enqueue the append kernel over T * Hkv rows.  new_f16: k_new/v_new are fp16
// (else bf16); cache_fp8: the cache holds fp8 e4m3fn codes (else new dtype).
hipError_t launch_append(const AppendArgs &a, bool new_f16, bool cache_fp8, hipStream_t stream);

// Arguments of the backward kernels (ua_backward.hip), passed by value.
struct BwdArgs {
    const void *q;                 // [T, Hq, 128]
    const void *k;                 // [Tk, Hkv, 128]
    const void *v;
    const void *o;                 // [T, Hq, 128] forward output
    const void *dout;              // [T, Hq, 128]
    const float *lse;              // [T, Hq] natural log
    const int32_t *cu_seqlens_q;   // [S + 1]
    const int32_t *cu_seqlens_k;   // [S + 1]
    void *dq;                      // [T, Hq, 128]
    void *dk;                      // [Tk, Hkv, 128]
    void *dv;
    float *lse2;                   // workspace [Hq][T]: LSE * log2(e) (+inf: row sees no key)
    float *delta;                  // workspace [Hq][T]: sum_d O dO
    int32_t num_seqs, num_tokens, num_tokens_k, num_q_heads, num_kv_heads;
    int32_t group;                 // Hq / Hkv
    int32_t block_q;               // dQ workgroup: query tokens (128 / G)
    int32_t q_slots;               // T / block_q + S
    int32_t dkdv_wgs;              // (Tk / 128 + S) * Hkv
    int32_t dq_wgs;                // q_slots * Hkv
    float scale;
};

// Enqueue the two backward kernels (dQ, which also forms Delta, then dK/dV) on stream.
hipError_t launch_backward(const BwdArgs &a, bool f16, bool causal, hipStream_t stream);

}  // namespace ua
