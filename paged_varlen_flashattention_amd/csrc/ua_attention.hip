// Unified paged, variable-length attention forward and split-KV combine for
// gfx950 (CDNA4).
//
// What is computed (page "flashatten takeaways EP2 工程", section "kv cache"):
// for every packed query row (token, query head) the softmax-weighted sum of
// the value rows of its sequence's cached keys, softmax(q K^T * scale) V.
// How it is organised:
//   * Work tiler.  One workgroup owns BLOCK_Q query tokens x the G query heads
//     of one kv head (GQA rows, page "vLLM Triton unified attention notes",
//     section kernel_unified_attention_2d) x one split.  The host sizes the
//     grid as (T / BLOCK_Q + S) query-block slots without reading device
//     memory; sequence s owns slots starting at cu[s] / BLOCK_Q + s, and each
//     workgroup finds its sequence by a binary search over cu_seqlens_q (same
//     section: find_seq_idx and the slot transform).
//   * Paged KV gather.  Key j of sequence s is slot j % bs of physical block
//     block_table[s][j / bs] (same section: four element strides).  A tile of
//     keys is gathered by the whole workgroup with 16-byte loads (one cache
//     row = 16 lanes), prefetched into registers one tile ahead, and staged in
//     LDS: K row-major, V transposed (d-major) so that both MFMA operands read
//     16 contiguous bytes per lane.  fp8 e4m3fn codes are widened to the q
//     dtype on the way in (exact), their scales folded into the score scale
//     and the epilogue.
//   * Contractions on MFMA 32x32x16 (bf16 or fp16 in, fp32 accumulate).  We
//     compute S^T = K Q^T, so each lane's accumulator column is one query row:
//     the row max and sum need one exchange between the two lane halves, the
//     rescale factor is a per-lane scalar, and the accumulator of S^T is, after
//     a fixed permutation of the K rows, directly the B operand of
//     O^T = V^T P^T.
//   * Online softmax (page "Fused Attention", FA2 tutorial listing, the inner
//     loop): running max m and sum l in log2 units, alpha = 2^(m_old - m_new)
//     rescales the accumulator, a single division at the end.  Unlike the
//     listing, m is only moved when a tile's max exceeds it by 2^8, so most
//     tiles skip the rescale.  Tiles that
//     every row of the block sees in full skip the mask (the tutorial's
//     off-band / on-band split).
//   * Split-KV (page "flashatten takeaways EP2 工程", section "源代码接口";
//     page "Fused Attention", section FlashDecoding): each split owns a
//     contiguous run of key tiles and stores a normalised fp32 partial and its
//     natural-log log-sum-exp; the combine kernel merges them.

#include "ua_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ua {
namespace {

constexpr int HD = kHeadSize;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kRescaleLog2 = 8.0f;     // lazy-rescale threshold, log2 units
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left at their
// maxima (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14])
constexpr int kWaitVmcnt0 = 0x0F70;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// D(32x32) += A(32x16) * B(16x32).  Lane l holds A row l%32 and B column l%32,
// 8 consecutive k per lane half; D column l%32, rows 8*(r/4) + 4*(l/32) + r%4.
template <bool F16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two fp32 -> two 16-bit floats (round to nearest even), low half first.
template <bool F16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    if constexpr (F16) {
        f16x2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        bf16x2 v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
}

// Eight fp8 e4m3fn codes -> eight 16-bit floats of the q dtype (exact: every
// e4m3fn value is representable in bf16 and in fp16).
template <bool F16>
__device__ __forceinline__ u32x4 widen_fp8(u32x2 v) {
    f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(v[0], false);
    f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(v[0], true);
    f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(v[1], false);
    f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(v[1], true);
    return u32x4{pack2<F16>(a[0], a[1]), pack2<F16>(b[0], b[1]), pack2<F16>(c[0], c[1]),
                 pack2<F16>(d[0], d[1])};
}

// A load the compiler must issue as a scalar (SMEM) load: the address is
// uniform across the wave and the data is read-only for the kernel's lifetime.
__device__ __forceinline__ int32_t sload(const int32_t *p) {
    return *(const __attribute__((address_space(4))) int32_t *)p;
}

// Swap bits 2 and 3 of a row index.  K row j of a 32-key block is fed to MFMA
// lane row swap23(j): then accumulator register r of lane half h holds key
// 16*(r/8) + 8*h + r%8, i.e. eight consecutive keys per register octet, which
// is exactly the k layout the P operand of the PV product needs.
__device__ __forceinline__ int swap23(int j) {
    return (j & ~12) | ((j >> 1) & 4) | ((j << 1) & 8);
}

// LDS swizzles (16-byte granules, XOR), K and V tiles both [TN][128] 16-bit:
//   K: granule g of key row j is stored at g ^ swz_k(j), so the 8 lanes that
//      read rows swap23(0..7) with one 16-byte read hit 8 distinct bank groups;
//   V: granule g of key row j is stored at g ^ swz_v(j); a transposing read
//      group covers 4 consecutive keys x 2 granules, which swz_v spreads over 8
//      distinct granule positions.
__device__ __forceinline__ int swz_k(int j) { return swap23(j & 15); }
__device__ __forceinline__ int swz_v(int j) { return (j & 3) << 1; }

typedef short s16x4 __attribute__((ext_vector_type(4)));

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds_row + 16*l (lds_row must be wave-uniform).  Issued as inline asm so
// the compiler does not guard every later LDS read with a wait for it; the
// kernel waits (wait_vmem) and synchronises (barrier) before it reads a stage
// that such loads filled.
// The global address is a wave-uniform base plus a per-lane 32-bit offset.
__device__ __forceinline__ void lds_dma16(const uint8_t *base, uint32_t lane_ofs, uint8_t *lds_row) {
    const uint32_t la = (uint32_t)reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) uint8_t *)(lds_row));
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(lane_ofs), "s"(base), "s"(la)
                 : "memory", "m0");
}

// Wait until every vector-memory load of this wave has completed (including
// loads that write LDS directly).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Transposing 8-byte LDS read (ds_read_b64_tr_b16).  Within each 16-lane
// group, lane i receives element i%4 of the 8 bytes addressed by lane 4e + i/4,
// for e = 0..3.
__device__ __forceinline__ s16x4 ds_read_tr16(const uint8_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(p));
}

// Two waves per SIMD: the kernel is written to fit 256 VGPRs so that the
// softmax of one wave overlaps the MFMAs of the other.
template <bool F16, bool FP8KV, bool CAUSAL, bool SPLIT, int NW, int TN>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(const AttnArgs a) {
    constexpr int NT = NW * 64;                 // threads
    constexpr int NKB = TN / 32;                // 32-key blocks per tile (S^T MFMA M)
    constexpr int NPV = TN / 16;                // 16-key steps per tile (PV MFMA K)
    constexpr int PAIRS = (TN / 2) * 16;        // (key pair, 8-d chunk) units per tile
    constexpr int PPT = PAIRS / NT;             // units per thread
    constexpr int KVB = FP8KV ? 1 : 2;          // bytes per cached element
    static_assert(PPT >= 1 && PAIRS % NT == 0, "tile / thread mismatch");
    using Chunk = typename std::conditional<FP8KV, u32x2, u32x4>::type;

    constexpr bool DB = NW > 1;                 // double-buffered LDS (prefill tile)
    constexpr bool DMA = DB && !FP8KV;          // K/V loaded straight into LDS
    constexpr int STAGE = 2 * TN * 256;         // bytes of one K + V stage
    // The two stages are separate objects so that alias analysis can tell an
    // LDS read of one stage from a direct-to-LDS load into the other.
    __shared__ __attribute__((aligned(16))) uint8_t lds[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[DB ? STAGE : 16];
    uint8_t *const ldsK = lds;
    uint8_t *const ldsV = lds + TN * 256;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hl = lane >> 5;                   // lane half
    const int lc = lane & 31;                   // accumulator column = query row in the wave

    // ---------------------------------------------------------------- tiler
    const int kvh = blockIdx.x % a.num_kv_heads;
    int slot = blockIdx.x / a.num_kv_heads;
    if (CAUSAL)
        slot = a.num_qslots - 1 - slot;         // late (long) query blocks first
    const int split = blockIdx.y;
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {                           // largest s with cu[s]/BLOCK_Q + s <= slot
        const int mid = (lo + hi + 1) >> 1;
        if (a.cu_seqlens_q[mid] / a.block_q + mid <= slot)
            lo = mid;
        else
            hi = mid - 1;
    }
    const int s = lo;
    const int cu0 = a.cu_seqlens_q[s];
    const int q_len = a.cu_seqlens_q[s + 1] - cu0;
    const int tq0 = (slot - (cu0 / a.block_q + s)) * a.block_q;
    if (tq0 >= q_len)
        return;                                 // empty slot (uniform, before any barrier)
    const int tq1 = min(q_len, tq0 + a.block_q);
    const int kv_len = a.seqused_k[s];
    const int ctx = kv_len - q_len;             // keys before the first query

    // keys seen by some row / by every row of this block
    const int kv_end = CAUSAL ? min(kv_len, ctx + tq1) : kv_len;
    const int full_end = CAUSAL ? min(kv_len, ctx + tq0 + 1) : kv_len;
    const int n_tiles = max(kv_end, 0) / TN + ((max(kv_end, 0) % TN) != 0);
    const int n_full = max(full_end, 0) / TN;
    int t_begin = 0, t_end = n_tiles;
    if (SPLIT) {
        const int per = (n_tiles + a.num_splits - 1) / a.num_splits;
        t_begin = min(n_tiles, split * per);
        t_end = min(n_tiles, t_begin + per);
    }

    // ---------------------------------------------------------------- rows
    const int G = a.group;
    const int r = wave * 32 + lc;
    const int tq = r / G;
    const int hg = r - tq * G;
    const int t_loc = tq0 + tq;
    const bool row_ok = t_loc < tq1;            // also false for rows past BLOCK_Q * G
    const int64_t tok = (int64_t)cu0 + t_loc;
    const int head = kvh * G + hg;
    const int lim = !row_ok ? 0 : (CAUSAL ? min(kv_len, ctx + t_loc + 1) : kv_len);
    const bool wave_on = wave * 32 < (tq1 - tq0) * G;

    // Q fragments: B operand of S^T = K Q^T, k-step ks covers d 16*ks .. 16*ks+15.
    u32x4 qf[8];
    if (row_ok) {
        const uint8_t *qp = (const uint8_t *)a.q + (tok * a.q_st_tok + (int64_t)head * a.q_st_head) * 2;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            qf[ks] = *(const u32x4 *)(qp + (16 * ks + 8 * hl) * 2);
    } else {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            qf[ks] = u32x4{0, 0, 0, 0};
    }
    // Q is resident before the key loop starts (a wait the compiler tracks, so
    // no later wait is spent on these loads)
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    // ---------------------------------------------------------------- loader
    // Thread unit i covers keys 2p, 2p+1 of the tile, p = tid/16 + i*NT/16,
    // and the d chunk c = tid%16 (d 8c .. 8c+7).  One load instruction of a
    // wave covers the 8-key group starting at rbase(i) = 8*wave + i*NT/8; a
    // page holds at least 16 keys, so the page of every load is wave-uniform:
    // its id is a scalar load of the block table and the page base is scalar
    // arithmetic, each lane adding a fixed offset (its key in the group, its d
    // chunk).  Page ids are fetched one tile ahead of the K/V loads that use
    // them, so no K/V load waits on a block-table load.
    const int c = tid & 15;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int lanep = 2 * ((tid >> 4) & 3);
    const int32_t *btrow = a.block_table + (int64_t)s * a.bt_stride;
    const int lbs = a.log2_block_size;
    const int bs_mask = (1 << lbs) - 1;
    const int last_page = (max(kv_end, 1) - 1) >> lbs;     // later table entries are never read
    const uint8_t *kbase = (const uint8_t *)a.k + (int64_t)kvh * a.kv_st_head * KVB;
    const uint8_t *vbase = (const uint8_t *)a.v + (int64_t)kvh * a.kv_st_head * KVB;
    const uint32_t lofs0 = (uint32_t)(lanep * a.kv_st_slot + 8 * c) * KVB;
    const uint32_t lofs1 = lofs0 + (uint32_t)a.kv_st_slot * KVB;
    int32_t blk_next[PPT];
    Chunk kr[PPT][2], vr[PPT][2];

    auto fetch_ids = [&](int tile) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int jb = tile * TN + 8 * wv + i * (NT / 8);
            blk_next[i] = sload(btrow + min(jb >> lbs, last_page));
        }
    };

    auto load_tile = [&](int tile) {           // page ids of `tile` are in blk_next
        const bool full = (tile + 1) * TN <= kv_end;
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int jb = tile * TN + 8 * wv + i * (NT / 8);
            const int64_t pofs =
                ((int64_t)blk_next[i] * a.kv_st_blk + (int64_t)(jb & bs_mask) * a.kv_st_slot) * KVB;
            const uint8_t *pk = kbase + pofs;
            const uint8_t *pv = vbase + pofs;
            Chunk k0 = *(const Chunk *)(pk + lofs0);
            Chunk k1 = *(const Chunk *)(pk + lofs1);
            Chunk v0 = *(const Chunk *)(pv + lofs0);
            Chunk v1 = *(const Chunk *)(pv + lofs1);
            if (!full) {
                // keys at or past kv_end were read from a clamped (allocated)
                // page; they must contribute nothing
                const int j0 = jb + lanep;
                if (j0 >= kv_end) { k0 = Chunk{}; v0 = Chunk{}; }
                if (j0 + 1 >= kv_end) { k1 = Chunk{}; v1 = Chunk{}; }
            }
            kr[i][0] = k0; kr[i][1] = k1;
            vr[i][0] = v0; vr[i][1] = v1;
        }
    };

    auto store_tile = [&](uint8_t *sK, uint8_t *sV) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = (tid >> 4) + i * (NT / 16);
            const int j0 = 2 * p, j1 = 2 * p + 1;
            u32x4 k0, k1, v0, v1;
            if constexpr (FP8KV) {
                k0 = widen_fp8<F16>(kr[i][0]); k1 = widen_fp8<F16>(kr[i][1]);
                v0 = widen_fp8<F16>(vr[i][0]); v1 = widen_fp8<F16>(vr[i][1]);
            } else {
                k0 = kr[i][0]; k1 = kr[i][1];
                v0 = vr[i][0]; v1 = vr[i][1];
            }
            *(u32x4 *)(sK + j0 * 256 + ((c ^ swz_k(j0)) << 4)) = k0;
            *(u32x4 *)(sK + j1 * 256 + ((c ^ swz_k(j1)) << 4)) = k1;
            *(u32x4 *)(sV + j0 * 256 + ((c ^ swz_v(j0)) << 4)) = v0;
            *(u32x4 *)(sV + j1 * 256 + ((c ^ swz_v(j1)) << 4)) = v1;
        }
    };

    // ---------------------------------------------------------------- compute
    const float c2 = a.scale_log2 * (FP8KV ? *a.k_scale : 1.0f);   // score -> log2 units
    f32x16 o[4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
        o[x] = f32x16{};
    float m = neg_inf();        // running max (log2 units, this row)
    float l = 0.0f;             // running sum over this lane half's keys

    auto compute_tile = [&](int tile, const uint8_t *sK, const uint8_t *sV) {
        // S^T (keys x rows) for each 32-key block
        f32x16 sacc[NKB];
#pragma unroll
        for (int b = 0; b < NKB; ++b)
            sacc[b] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int b = 0; b < NKB; ++b) {
                const uint8_t *krow = sK + (32 * b + swap23(lc)) * 256;
                const u32x4 kf = *(const u32x4 *)(krow + (((2 * ks + hl) ^ (lane & 15)) << 4));
                sacc[b] = mfma32<F16>(kf, qf[ks], sacc[b]);
            }

        // mask (boundary / diagonal tiles only) and row max
        if (tile >= n_full) {
            const int j0 = tile * TN + 8 * hl;
#pragma unroll
            for (int b = 0; b < NKB; ++b)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int j = j0 + 32 * b + 16 * (q >> 3) + (q & 7);
                    if (j >= lim)
                        sacc[b][q] = neg_inf();
                }
        }
        float mx = neg_inf();
#pragma unroll
        for (int b = 0; b < NKB; ++b)
#pragma unroll
            for (int q = 0; q < 16; ++q)
                mx = fmaxf(mx, sacc[b][q]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));

        // The reference max m only moves when this tile's max exceeds it by
        // more than kRescaleLog2 (a factor 2^8): weights 2^(s - m) then stay
        // below 256, and the accumulator and sum are rescaled only on those
        // (rare, after the first tiles) steps.  The final division by l makes
        // the result independent of which reference was used.
        const float tmax = mx * c2;
        const bool grow = tmax > m + kRescaleLog2;          // also true for the first finite max
        if (__ballot(grow) != 0) {
            // rows that do not grow keep alpha = 1 (their m may still be -inf)
            const float alpha = grow ? __builtin_amdgcn_exp2f(m - tmax) : 1.0f;  // 0 if m was -inf
            m = grow ? tmax : m;
            l *= alpha;
#pragma unroll
            for (int x = 0; x < 4; ++x)
                o[x] *= alpha;
        }
        const float m_use = (m == neg_inf()) ? 0.0f : m;    // fully masked so far: weights 0
        // weights and their fp32 row sum (four partial sums for ILP)
        float rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int b = 0; b < NKB; ++b)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[b][q], c2, -m_use));
                sacc[b][q] = p;
                rs[q & 3] += p;
            }
        l += (rs[0] + rs[1]) + (rs[2] + rs[3]);

        // P (16-bit) as the B operand of O^T += V^T P^T
        u32x4 pf[NPV];
#pragma unroll
        for (int b = 0; b < NKB; ++b)
#pragma unroll
            for (int hsel = 0; hsel < 2; ++hsel) {
                const int q0 = 8 * hsel;
                pf[2 * b + hsel] = u32x4{pack2<F16>(sacc[b][q0 + 0], sacc[b][q0 + 1]),
                                         pack2<F16>(sacc[b][q0 + 2], sacc[b][q0 + 3]),
                                         pack2<F16>(sacc[b][q0 + 4], sacc[b][q0 + 5]),
                                         pack2<F16>(sacc[b][q0 + 6], sacc[b][q0 + 7])};
            }
        // V^T fragment of 16-lane group g = lane/16 (d 32x + 16(g&1) .. +15,
        // keys 16kk + 8(g>>1) .. +7) by two transposing LDS reads: lane j of the
        // group points at key +4t + j/4, d +4(j%4) .. +3, and receives
        // V[key + 4t + e][d + j] for e = 0..3.
        const int jg = lane & 15;
        const int vrow0 = 8 * hl + (jg >> 2);                // key within a 16-key step
        const int vsw = swz_v(vrow0);
#pragma unroll
        for (int kk = 0; kk < NPV; ++kk)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int gran = 4 * x + 2 * ((lane >> 4) & 1) + ((jg & 3) >> 1);
                const uint8_t *va = sV + (16 * kk + vrow0) * 256 + ((gran ^ vsw) << 4) + 8 * (jg & 1);
                const s16x4 r0 = ds_read_tr16(va);
                const s16x4 r1 = ds_read_tr16(va + 4 * 256);
                const u32x2 w0 = __builtin_bit_cast(u32x2, r0);
                const u32x2 w1 = __builtin_bit_cast(u32x2, r1);
                o[x] = mfma32<F16>(u32x4{w0[0], w0[1], w1[0], w1[1]}, pf[kk], o[x]);
            }
    };

    // ---------------------------------------------------------------- main loop
    if constexpr (DMA) {
        // 16-bit caches, prefill tile: K/V go straight from HBM into LDS
        // (global_load_lds, 16 bytes per lane), no register staging.  Wave w
        // fills keys 16w .. 16w+15 of the tile (one page) with four 4-key
        // instructions per tensor; lane l of an instruction lands at LDS byte
        // 16*l of those 4 rows, so it fetches the d chunk whose swizzled
        // position that is.  Two LDS stages: the DMA of tile + 1 runs under
        // the compute of tile; one barrier per tile.
        static_assert(TN / NW == 16, "one 16-key chunk per wave");
        uint8_t *const sK1 = lds_b;
        uint8_t *const sV1 = lds_b + TN * 256;
        const int lrow = lane >> 4;                           // row within a 4-key group
        const uint32_t rofs = (uint32_t)(lrow * a.kv_st_slot * KVB);
        uint32_t koff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            koff[i] = rofs + (uint32_t)(((lane & 15) ^ swz_k(4 * i + lrow)) << 4);
        const uint32_t voff = rofs + (uint32_t)(((lane & 15) ^ swz_v(lrow)) << 4);
        const int wrow = 16 * wv;                             // this wave's first key in the tile
        int32_t blk_dma = 0;
        auto fetch_id = [&](int tile) {
            blk_dma = sload(btrow + min((tile * TN + wrow) >> lbs, last_page));
        };
        auto dma_tile = [&](int tile, uint8_t *sK, uint8_t *sV) {
            const int j = tile * TN + wrow;
            const int64_t pofs =
                ((int64_t)blk_dma * a.kv_st_blk + (int64_t)(j & bs_mask) * a.kv_st_slot) * KVB;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t gofs = pofs + (int64_t)(4 * i) * a.kv_st_slot * KVB;
                lds_dma16(kbase + gofs, koff[i], sK + (wrow + 4 * i) * 256);
                lds_dma16(vbase + gofs, voff, sV + (wrow + 4 * i) * 256);
            }
        };
        // keys at or past kv_end came from a clamped (allocated) page: zero
        // their V rows so that weight 0 times whatever was there stays 0
        auto zero_tail = [&](int tile, uint8_t *sV) {
            if ((tile + 1) * TN > kv_end) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (tile * TN + wrow + 4 * i + lrow >= kv_end)
                        *(u32x4 *)(sV + (wrow + 4 * i) * 256 + 16 * lane) = u32x4{0, 0, 0, 0};
            }
        };
        if (t_begin < t_end) {
            fetch_id(t_begin);
            dma_tile(t_begin, ldsK, ldsV);
            if (t_begin + 1 < t_end)
                fetch_id(t_begin + 1);
            wait_vmem();
            zero_tail(t_begin, ldsV);
            __syncthreads();
        }
        auto step = [&](int tile, uint8_t *cK, uint8_t *cV, uint8_t *nK, uint8_t *nV) {
            if (tile + 1 < t_end) {
                dma_tile(tile + 1, nK, nV);
                if (tile + 2 < t_end)
                    fetch_id(tile + 2);
            }
            if (wave_on)
                compute_tile(tile, cK, cV);
            if (tile + 1 < t_end) {
                wait_vmem();
                zero_tail(tile + 1, nV);
                __syncthreads();
            }
        };
        for (int tile = t_begin; tile < t_end; tile += 2) {
            step(tile, ldsK, ldsV, sK1, sV1);
            if (tile + 1 < t_end)
                step(tile + 1, sK1, sV1, ldsK, ldsV);
        }
    } else if constexpr (DB) {
        // Two LDS buffers: compute(tile) reads one while the other receives
        // tile + 1; one barrier per tile.
        uint8_t *const sK1 = lds_b;
        uint8_t *const sV1 = lds_b + TN * 256;
        if (t_begin < t_end) {
            fetch_ids(t_begin);
            load_tile(t_begin);
            if (t_begin + 1 < t_end)
                fetch_ids(t_begin + 1);
            store_tile(ldsK, ldsV);
            __syncthreads();
            if (t_begin + 1 < t_end) {
                load_tile(t_begin + 1);
                if (t_begin + 2 < t_end)
                    fetch_ids(t_begin + 2);
            }
        }
        // unrolled by two so that each stage's LDS addresses are constants
        auto step = [&](int tile, uint8_t *cK, uint8_t *cV, uint8_t *nK, uint8_t *nV) {
            if (wave_on)
                compute_tile(tile, cK, cV);
            if (tile + 1 < t_end) {
                store_tile(nK, nV);
                __syncthreads();
                if (tile + 2 < t_end) {
                    load_tile(tile + 2);
                    if (tile + 3 < t_end)
                        fetch_ids(tile + 3);
                }
            }
        };
        for (int tile = t_begin; tile < t_end; tile += 2) {
            step(tile, ldsK, ldsV, sK1, sV1);
            if (tile + 1 < t_end)
                step(tile + 1, sK1, sV1, ldsK, ldsV);
        }
    } else {
        if (t_begin < t_end) {
            fetch_ids(t_begin);
            load_tile(t_begin);
            if (t_begin + 1 < t_end)
                fetch_ids(t_begin + 1);
        }
        for (int tile = t_begin; tile < t_end; ++tile) {
            __syncthreads();        // previous tile fully consumed
            store_tile(ldsK, ldsV);
            __syncthreads();        // tile visible to every wave
            if (tile + 1 < t_end) {
                load_tile(tile + 1);
                if (tile + 2 < t_end)
                    fetch_ids(tile + 2);
            }
            if (wave_on)
                compute_tile(tile, ldsK, ldsV);
        }
    }

    // ---------------------------------------------------------------- epilogue
    if (!wave_on)
        return;
    const float l_row = l + __shfl_xor(l, 32);
    if (!row_ok)
        return;
    const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
    const float lse = l_row > 0.0f ? m * kLn2 + __logf(l_row) : neg_inf();
    const float sc = inv * (FP8KV ? *a.v_scale : 1.0f);
    if constexpr (!SPLIT) {
        uint8_t *op = (uint8_t *)a.out + (tok * a.o_st_tok + (int64_t)head * a.o_st_head) * 2;
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * x + 8 * g + 4 * hl;
                const u32x2 w = {pack2<F16>(o[x][4 * g] * sc, o[x][4 * g + 1] * sc),
                                 pack2<F16>(o[x][4 * g + 2] * sc, o[x][4 * g + 3] * sc)};
                *(u32x2 *)(op + d * 2) = w;
            }
        if (a.lse_out != nullptr && hl == 0)
            a.lse_out[tok * a.num_q_heads + head] = lse;
    } else {
        const int64_t row = ((int64_t)split * a.num_tokens + tok) * a.num_q_heads + head;
        float *op = a.o_part + row * HD;
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * x + 8 * g + 4 * hl;
                *(f32x4 *)(op + d) = f32x4{o[x][4 * g] * sc, o[x][4 * g + 1] * sc,
                                           o[x][4 * g + 2] * sc, o[x][4 * g + 3] * sc};
            }
        if (hl == 0)
            a.lse_part[row] = lse;
    }
}

// One 32-lane half-wave per row; lane i owns d 4i .. 4i+3.
template <bool F16>
__global__ __launch_bounds__(256) void combine_kernel(const float *o_part, const float *lse_part,
                                                      int32_t P, int64_t rows, int32_t Hq, void *out,
                                                      int64_t o_st_tok, int64_t o_st_head,
                                                      float *lse_out) {
    const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
    if (row >= rows)
        return;
    const int i = threadIdx.x & 31;
    float L = neg_inf();
    for (int p = 0; p < P; ++p)
        L = fmaxf(L, lse_part[(int64_t)p * rows + row]);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float wsum = 0.0f;
    if (L != neg_inf()) {
        for (int p = 0; p < P; ++p) {
            const int64_t pr = (int64_t)p * rows + row;
            const float w = __builtin_amdgcn_exp2f((lse_part[pr] - L) * kLog2e);
            const f32x4 v = *(const f32x4 *)(o_part + pr * HD + 4 * i);
            acc += w * v;
            wsum += w;
        }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    const int64_t tok = row / Hq;
    const int64_t head = row - tok * Hq;
    uint8_t *op = (uint8_t *)out + (tok * o_st_tok + head * o_st_head + 4 * i) * 2;
    *(u32x2 *)op = u32x2{pack2<F16>(acc[0] * inv, acc[1] * inv), pack2<F16>(acc[2] * inv, acc[3] * inv)};
    if (lse_out != nullptr && i == 0)
        lse_out[row] = wsum > 0.0f ? L + __logf(wsum) : neg_inf();
}

template <bool F16, bool FP8KV, bool CAUSAL, bool SPLIT>
hipError_t launch_tile(const AttnArgs &a, Tile tile, dim3 grid, hipStream_t st) {
    if (tile == Tile::Prefill)
        hipLaunchKernelGGL((attn_fwd_kernel<F16, FP8KV, CAUSAL, SPLIT, 4, 64>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((attn_fwd_kernel<F16, FP8KV, CAUSAL, SPLIT, 1, 32>), grid, dim3(64), 0, st, a);
    return hipGetLastError();
}

template <bool F16, bool FP8KV>
hipError_t launch_mode(const AttnArgs &a, Tile tile, bool causal, bool split, dim3 grid, hipStream_t st) {
    if (causal)
        return split ? launch_tile<F16, FP8KV, true, true>(a, tile, grid, st)
                     : launch_tile<F16, FP8KV, true, false>(a, tile, grid, st);
    return split ? launch_tile<F16, FP8KV, false, true>(a, tile, grid, st)
                 : launch_tile<F16, FP8KV, false, false>(a, tile, grid, st);
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, Tile tile, bool q_f16, bool kv_fp8, bool causal,
                            bool split, dim3 grid, hipStream_t stream) {
    if (q_f16)
        return kv_fp8 ? launch_mode<true, true>(a, tile, causal, split, grid, stream)
                      : launch_mode<true, false>(a, tile, causal, split, grid, stream);
    return kv_fp8 ? launch_mode<false, true>(a, tile, causal, split, grid, stream)
                  : launch_mode<false, false>(a, tile, causal, split, grid, stream);
}

hipError_t launch_combine(const float *o_part, const float *lse_part, int32_t num_splits,
                          int64_t rows, int32_t num_q_heads, void *out, bool out_f16,
                          int64_t o_st_tok, int64_t o_st_head, float *lse_out, hipStream_t stream) {
    const dim3 grid((unsigned)((rows + 7) / 8));
    if (out_f16)
        hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, stream, o_part, lse_part,
                           num_splits, rows, num_q_heads, out, o_st_tok, o_st_head, lse_out);
    else
        hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, stream, o_part, lse_part,
                           num_splits, rows, num_q_heads, out, o_st_tok, o_st_head, lse_out);
    return hipGetLastError();
}

}  // namespace ua
