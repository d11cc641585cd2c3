// KV-cache append for gfx950: the new tokens' k and v rows written into their
// page slots (page "flashatten takeaways EP2 工程", section "kv cache": the
// cache of a sequence grows by the new rows, K_{1:t+1} = [K_{1:t}; k_{t+1}];
// page "vLLM Triton unified attention notes", section
// kernel_unified_attention_2d: key position j of sequence s is slot j % bs of
// block block_table[s][j / bs], addressed through the cache's four strides).
//
// One 16-lane group per (token, kv head) row; lane c moves the 16 bytes of d
// 8c .. 8c+7 of the 128-element row (256 contiguous bytes of k_new / v_new and
// of a 16-bit cache row: coalesced on both sides).  An fp8 cache receives 8
// codes per lane (the row's 128 bytes): each value is divided by the tensor's
// scale, saturated to +-448 and rounded to the nearest e4m3fn code, ties to
// even (v_cvt_pk_fp8_f32, OCP e4m3fn on gfx950).

#include "ua_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ua {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kRowsPerGroup = 16;     // rows per 256-thread workgroup

// Eight values of the new row -> eight e4m3fn codes (saturating, RNE).
template <bool F16>
__device__ __forceinline__ u32x2 to_fp8(u32x4 raw, float scale) {
    float x[8];
    if constexpr (F16) {
        const f16x8 h = __builtin_bit_cast(f16x8, raw);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            x[e] = (float)h[e];
    } else {
        const bf16x8 h = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            x[e] = (float)h[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
        x[e] = fminf(fmaxf(x[e] / scale, -448.0f), 448.0f);
    u32x2 out;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        uint32_t word = 0;
        word = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w + 0], x[4 * w + 1], (int)word, false);
        word = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w + 2], x[4 * w + 3], (int)word, true);
        out[w] = word;
    }
    return out;
}

template <bool F16, bool FP8>
__global__ __launch_bounds__(256) void kv_append_kernel(const AppendArgs a) {
    const int64_t row = (int64_t)blockIdx.x * kRowsPerGroup + (threadIdx.x >> 4);
    const int c = threadIdx.x & 15;
    if (row >= (int64_t)a.num_tokens * a.num_kv_heads)
        return;
    const int t = (int)(row / a.num_kv_heads);
    const int h = (int)(row - (int64_t)t * a.num_kv_heads);
    if (t >= a.cu_seqlens_q[a.num_seqs])
        return;                                 // token of no sequence
    int lo = 0, hi = a.num_seqs - 1;            // largest s with cu[s] <= t
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.cu_seqlens_q[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    const int s = lo;
    const int q_len = a.cu_seqlens_q[s + 1] - a.cu_seqlens_q[s];
    const int pos = a.seqused_k[s] - q_len + (t - a.cu_seqlens_q[s]);
    const int32_t blk = a.block_table[(int64_t)s * a.bt_stride + (pos >> a.log2_block_size)];
    const int slot = pos & ((1 << a.log2_block_size) - 1);
    const int64_t src = (int64_t)t * a.new_st_tok + (int64_t)h * a.new_st_head + 8 * c;      // elements
    const int64_t dst = (int64_t)blk * a.kv_st_blk + (int64_t)slot * a.kv_st_slot +
                        (int64_t)h * a.kv_st_head + 8 * c;                                   // elements
    const u32x4 kr = *(const u32x4 *)((const uint16_t *)a.k_new + src);
    const u32x4 vr = *(const u32x4 *)((const uint16_t *)a.v_new + src);
    if constexpr (FP8) {
        *(u32x2 *)((uint8_t *)a.k_cache + dst) = to_fp8<F16>(kr, *a.k_scale);
        *(u32x2 *)((uint8_t *)a.v_cache + dst) = to_fp8<F16>(vr, *a.v_scale);
    } else {
        *(u32x4 *)((uint16_t *)a.k_cache + dst) = kr;
        *(u32x4 *)((uint16_t *)a.v_cache + dst) = vr;
    }
}

template <bool F16, bool FP8>
hipError_t launch(const AppendArgs &a, hipStream_t st) {
    const int64_t rows = (int64_t)a.num_tokens * a.num_kv_heads;
    const dim3 grid((unsigned)((rows + kRowsPerGroup - 1) / kRowsPerGroup));
    (void)hipGetLastError();                    // report this launch's status only
    hipLaunchKernelGGL((kv_append_kernel<F16, FP8>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, bool new_f16, bool cache_fp8, hipStream_t stream) {
    if (new_f16)
        return cache_fp8 ? launch<true, true>(a, stream) : launch<true, false>(a, stream);
    return cache_fp8 ? launch<false, true>(a, stream) : launch<false, false>(a, stream);
}

}  // namespace ua
