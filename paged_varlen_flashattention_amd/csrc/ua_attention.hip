// Unified paged, variable-length attention forward and split-KV combine for
// gfx950 (CDNA4).
//
// What is computed (page "flashatten takeaways EP2 工程", section "kv cache"):
// for every packed query row (token, query head) the softmax-weighted sum of
// the value rows of its sequence's cached keys, softmax(q K^T * scale) V.
//
// One attention kernel (attn_fwd_kernel) runs two workgroup bodies in one
// launch, sharing one per-tile step:
//   * prefill_body: one workgroup of 4 waves owns BLOCK_Q = 128 / G
//     query tokens x the G query heads of one kv head (GQA rows, page "vLLM
//     Triton unified attention notes", section kernel_unified_attention_2d)
//     x one split; each wave owns 32 of the 128 rows and all waves share each
//     64-key tile staged in LDS.  The host sizes the grid as (T / BLOCK_Q + S)
//     query-block slots without reading device memory; sequence s owns the
//     slots from cu[s] / BLOCK_Q + s, and each workgroup finds its sequence by
//     a binary search over cu_seqlens_q (same section: find_seq_idx and the
//     slot transform).
//     Split launches with prefill work (few query blocks per kv head) use
//     8-wave workgroups instead: two such 4-wave key groups take alternate
//     tiles of the split, each with its own LDS stages and its own LDS-counter
//     barrier, and merge their softmax states at the end.
//   * decode_body: sequences whose q_len * G rows fit one wave (<= 32).
//     One workgroup per (sequence, kv head, split); its 4 (or 8) waves hold
//     the same rows and stream disjoint 32-key units of the key range
//     independently (K and V rows loaded whole into wave-private LDS stages),
//     then merge their partial softmax states at the end.  No barrier in the
//     key loop, so each wave keeps its own loads in flight.
//
// The per-tile step (attend_tile):
//   * MFMA 32x32x16 (bf16 or fp16 in, fp32 accumulate) computing S^T = K Q^T,
//     so each lane's accumulator column is one query row: the row max and sum
//     need one exchange between the two lane halves, the rescale factor is a
//     per-lane scalar, and the accumulator of S^T is, after a fixed permutation
//     of the K rows, directly the B operand of O^T = V^T P^T;
//   * online softmax (page "Fused Attention", FA2 tutorial listing, the inner
//     loop): running max m and sum l in log2 units, a single division at the
//     end.  Unlike the listing, m only moves when a tile's max exceeds it by
//     2^8, so most tiles skip the accumulator rescale; tiles that every row
//     sees in full skip the mask (the tutorial's off-band / on-band split).
//
// Paged KV gather: key j of sequence s is slot j % bs of physical block
// block_table[s][j / bs] (page "vLLM Triton unified attention notes", section
// kernel_unified_attention_2d: four element strides).  fp8 e4m3fn codes are
// widened to the q dtype (exact): the prefill body keeps a tile's codes in LDS
// and widens each operand fragment as it reads it, the decode body widens on
// the way into LDS; k_scale is folded into the score scale and v_scale into
// the epilogue.
//
// Split-KV (page "flashatten takeaways EP2 工程", section "源代码接口"; page
// "Fused Attention", section FlashDecoding): each split owns a contiguous run
// of key tiles and stores a normalised fp32 partial and its natural-log
// log-sum-exp; combine_kernel merges them.

#include "ua.h"
#include "ua_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
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
// decode merge record per lane: 64 accumulator values, m, l
constexpr int kDecodeMergeRows = 4 * 16 + 2;
// LDS of one workgroup of nw waves: the larger of the prefill stages (two K
// and two V tiles of 64 keys per 4-wave key group, then two key-group barrier
// counters) and the merge records (decode: nw waves x 66 x 64 floats; two
// prefill key groups need 4 waves')
constexpr int lds_bytes(int nw) {
    return ((nw / 4) * 2 * 2 * 64 * 256 + 16) > (nw * kDecodeMergeRows * 64 * 4)
               ? ((nw / 4) * 2 * 2 * 64 * 256 + 16)
               : (nw * kDecodeMergeRows * 64 * 4);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

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

// Eight fp8 e4m3fn codes -> eight 16-bit floats of the q dtype, one
// conversion per pair (v_cvt_scalef32_pk_{bf16,f16}_fp8 with scale 1: exact,
// since every e4m3fn value is representable in bf16 and in fp16).
template <bool F16>
__device__ __forceinline__ u32x4 widen_fp8(u32x2 v) {
    if constexpr (F16) {
        return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[0], 1.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[0], 1.0f, true)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[1], 1.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[1], 1.0f, true))};
    } else {
        return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, true)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, true))};
    }
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

// LDS swizzles (16-byte granules, XOR), K and V tiles both [keys][128] 16-bit.
// The LDS serves 256 bytes (64 banks) per clock: a 16-byte read is served 16
// lanes at a time, an 8-byte read 32 lanes at a time, and a pass is free of
// bank conflicts when its lanes cover the 16 granule positions of a 256-byte
// row once each.
//   K: granule g of key row j is stored at g ^ swz_k(j), so the 16 lanes that
//      read rows swap23(0..15) with one 16-byte read hit 16 distinct positions;
//   V: granule g of key row j is stored at g ^ swz_v(j); the 32 lanes of a
//      transposing read cover 4 consecutive keys x 4 consecutive granules
//      (4x .. 4x+3), and swz_v moves each of the 4 keys to its own group of 4
//      positions.
__device__ __forceinline__ int swz_k(int j) { return swap23(j & 15); }
__device__ __forceinline__ int swz_v(int j) { return (j & 3) << 2; }

// Transposing 8-byte LDS read (ds_read_b64_tr_b16).  Within each 16-lane
// group, lane i receives element i%4 of the 8 bytes addressed by lane 4e + i/4,
// for e = 0..3.
__device__ __forceinline__ s16x4 ds_read_tr16(const uint8_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(p));
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds_row + 16*l (lds_row must be wave-uniform); the global address is a
// wave-uniform base plus a per-lane 32-bit offset.  Issued as inline asm so
// the compiler does not guard every later LDS read with a wait for it; the
// kernel waits (wait_vmem) and synchronises (barrier) before it reads a stage
// that such loads filled.
__device__ __forceinline__ void lds_dma16(const uint8_t *base, uint32_t lane_ofs, uint8_t *lds_row) {
    const uint32_t la = (uint32_t)reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) uint8_t *)(lds_row));
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(lane_ofs), "s"(base), "s"(la)
                 : "memory", "m0");
}

// As lds_dma16, with the LDS row given as a wave-uniform base plus a
// compile-time byte offset added in the same asm block (s_add_u32 m0), so the
// compiler keeps one scalar base instead of one register per row address (the
// 16 row addresses of a tile's loads otherwise spill to VGPR lanes and are
// reloaded every tile).  s_add_u32 writes SCC, hence the "scc" clobber: the
// compiler must not keep a carry (the high half of a 64-bit add) or a branch
// condition live across this block.
template <int OFS>
__device__ __forceinline__ void lds_dma16_at(const uint8_t *base, uint32_t lane_ofs, uint32_t lds_base) {
    asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(lane_ofs), "s"(base), "s"(lds_base), "i"(OFS)
                 : "memory", "m0", "scc");
}

// Combine a value with the one held by the lane 32 positions away (the other
// half of the wave), on every lane: v_permlane32_swap exchanges the halves of
// two registers, so with both operands equal to v the two results hold v and
// its partner in some order, and a commutative op of them is the same on both
// halves.  No LDS round trip, unlike a shuffle.
__device__ __forceinline__ float xhalf_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wait until every vector-memory load of this wave has completed (including
// loads that write LDS directly).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// D(32x32) += A(32x64) * B(64x32), fp8 e4m3 operands, unit block scales.
// Lane l holds A row (B column) l % 32 and the 32 bytes k = 32 (l / 32) .. +31
// of it; D as in mfma32.
__device__ __forceinline__ f32x16 mfma32_f8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Four fp32 values -> four e4m3fn codes, x0 in the low byte (round to
// nearest even).
__device__ __forceinline__ uint32_t pack_fp8x4(float x0, float x1, float x2, float x3) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, lo, true);
}

// Barrier of the 4 waves of one key group of a two-group prefill workgroup, so
// that the groups do not run in lock step (one hardware barrier per workgroup
// would align their MFMA and softmax phases on every SIMD).  One LDS counter
// per group: a wave adds 1 once its own LDS writes are complete (its direct
// loads into LDS were waited for before), then polls until the counter reaches
// target = 4 x (barriers so far).  Every wave of a group passes the same
// sequence of barriers, so the wait ends; the poll count is bounded all the
// same (spin_limit polls), so that a wave can never spin forever.  Returns
// true when the limit was reached first: the wave then went on without the
// barrier's guarantee, and the workgroup marks its outputs NaN (see
// mark_lost / poison_row), so a timed-out wait never yields a silently wrong
// result.
__device__ __forceinline__ bool group_barrier(uint32_t *ctr, uint32_t target, int lane, int spin_limit) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0)
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    bool reached = false;
    for (int i = 0; i < spin_limit; ++i) {
        if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) {
            reached = true;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
    return !reached;
}

// A wave whose key-group barrier timed out sets the workgroup's lost flag (an
// LDS word next to the barrier counters); the epilogue reads it after a full
// workgroup barrier.
__device__ __forceinline__ void mark_lost(uint32_t *flag, bool lost, int lane) {
    if (lost && lane == 0)
        __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ------------------------------------------------------------------ per-tile step

// Online-softmax state of one wave's 32 query rows (row = accumulator column
// lane % 32; both lane halves hold the same row).
struct RowState {
    f32x16 o[4];   // O^T: block x, register r -> d = 32x + 8(r/4) + 4(lane/32) + r%4
    float m;       // reference max, log2 units (-inf until the row sees a key)
    float l;       // sum of weights of this lane half's keys, relative to m
};

__device__ __forceinline__ void init_rows(RowState &st) {
#pragma unroll
    for (int x = 0; x < 4; ++x)
        st.o[x] = f32x16{};
    st.m = neg_inf();
    st.l = 0.0f;
}

// One tile of 32*NKB keys against the wave's 32 query rows, in three steps
// (scores, softmax weights, PV product) that attend_tile runs back to back
// and the ping-pong prefill body runs in different phases.
//   kfrag(b, ks): K A-operand of key block b (MFMA row i = key 32b + swap23(i)),
//                 d 16ks .. 16ks+15 (8 per lane half);
//   vfrag(kk, x): V^T A-operand of d block x (row i = d 32x + i) for keys
//                 16kk .. 16kk+15, slot s of lane half h = key 16kk + 8h + s;
//   key0:  absolute index of the tile's first key;
//   masked: apply the per-row visibility limit lim (keys >= lim get weight 0).

// S^T of the tile (sacc[b] = key block b).  HOIST: every K fragment of the
// tile is read from LDS before the first MFMA (the chain then waits for its
// operands once instead of an LDS latency every step; 8 * NKB * 4 more live
// registers, so only where the register file has room).
template <bool F16, int NKB, bool HOIST, class KF>
__device__ __forceinline__ void tile_scores(f32x16 (&sacc)[NKB], const u32x4 (&qf)[8], KF kfrag) {
#pragma unroll
    for (int b = 0; b < NKB; ++b)
        sacc[b] = f32x16{};
    u32x4 kall[HOIST ? 8 : 1][HOIST ? NKB : 1];
    if constexpr (HOIST) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int b = 0; b < NKB; ++b)
                kall[ks][b] = kfrag(b, ks);
    }
    // the score MFMA chain runs at raised wave priority: when the matrix
    // pipe frees up, this wave's next MFMA issues ahead of the softmax VALU
    // work of the other wave on the SIMD
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int b = 0; b < NKB; ++b) {
            if constexpr (HOIST)
                sacc[b] = mfma32<F16>(kall[ks][b], qf[ks], sacc[b]);
            else
                sacc[b] = mfma32<F16>(kfrag(b, ks), qf[ks], sacc[b]);
        }
    __builtin_amdgcn_s_setprio(0);
}

// Per-row extras of the local-attention / ALiBi path (page "flashatten
// takeaways EP2 工程", section "源代码接口": the window and ALiBi switches of the
// FA2 forward launch): the first visible key (keys below it are masked like
// those at or past lim) and the ALiBi term -slope * |pos - j| in log2 units.
struct RowExt {
    int lo;        // first visible key of the row
    int pos;       // absolute position of the row's query (below 2^24: exact in fp32)
    float sl2;     // ALiBi slope * log2(e) (0 without ALiBi)
};

// Mask, row max, (lazy) rescale of the state, weights and their row sum; the
// weights leave as the 16-bit B operand pf of O^T += V^T P^T.  EXT: also the
// lower bound of a local window and, when alibi, the ALiBi term (added to the
// scaled score before the row max).
template <bool F16, int NKB, bool EXT = false>
__device__ __forceinline__ void tile_softmax(RowState &st, f32x16 (&sacc)[NKB], u32x4 (&pf)[2 * NKB],
                                             int key0, bool masked, int lim, float c2, int lane,
                                             RowExt ext = RowExt{0, 0, 0.0f}, bool alibi = false) {
    const int hl = lane >> 5;
    // mask (boundary / diagonal tiles only) and row max
    if (masked) {
        const int j0 = key0 + 8 * hl;
#pragma unroll
        for (int b = 0; b < NKB; ++b)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int j = j0 + 32 * b + 16 * (q >> 3) + (q & 7);
                if (j >= lim || (EXT && j < ext.lo))
                    sacc[b][q] = neg_inf();
            }
    }
    if constexpr (EXT) {
        if (alibi) {                            // uniform: the launch has slopes
            // scaled score with the bias, in log2 units; the rest then runs
            // with a unit scale
            const int base = ext.pos - (key0 + 8 * hl);
            const float nsl2 = -ext.sl2;
#pragma unroll
            for (int b = 0; b < NKB; ++b)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int d = base - (32 * b + 16 * (q >> 3) + (q & 7));
                    sacc[b][q] = __builtin_fmaf(nsl2, __builtin_fabsf((float)d), sacc[b][q] * c2);
                    if ((q & 3) == 3)
                        __builtin_amdgcn_sched_barrier(0);   // keep the temporaries few
                }
            c2 = 1.0f;
        }
    }
    float mx = neg_inf();
#pragma unroll
    for (int b = 0; b < NKB; ++b)
#pragma unroll
        for (int q = 0; q < 16; ++q)
            mx = fmaxf(mx, sacc[b][q]);
    mx = xhalf_max(mx);

    // The reference max m only moves when this tile's max exceeds it by more
    // than kRescaleLog2 (a factor 2^8): weights 2^(s - m) then stay below 256,
    // and the accumulator and sum are rescaled only on those (rare, after the
    // first tiles) steps.  The final division by l makes the result
    // independent of which reference was used.
    const float tmax = mx * c2;
    const bool grow = tmax > st.m + kRescaleLog2;           // also true for the first finite max
    if (__ballot(grow) != 0) {
        // rows that do not grow keep alpha = 1 (their m may still be -inf)
        const float alpha = grow ? __builtin_amdgcn_exp2f(st.m - tmax) : 1.0f;  // 0 if m was -inf
        st.m = grow ? tmax : st.m;
        st.l *= alpha;
#pragma unroll
        for (int x = 0; x < 4; ++x)
            st.o[x] *= alpha;
    }
    const float m_use = (st.m == neg_inf()) ? 0.0f : st.m;  // fully masked so far: weights 0
    // weights, P (16-bit) as the B operand of O^T += V^T P^T, and the row sum
    // (four partial sums for ILP).  fp16: the sum is taken over the rounded
    // fp16 weights the PV product uses (one v_dot2 per pair, fp32
    // accumulation: half the instructions of fp32 adds); bf16: over the fp32
    // weights (bf16 rounding of the sum's terms would cost ~2^-9 of the
    // log-sum-exp).
    float rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int b = 0; b < NKB; ++b)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[b][q], c2, -m_use));
            sacc[b][q] = p;
            if constexpr (!F16)
                rs[q & 3] += p;
        }
#pragma unroll
    for (int b = 0; b < NKB; ++b)
#pragma unroll
        for (int hsel = 0; hsel < 2; ++hsel) {
            const int q0 = 8 * hsel;
            if constexpr (F16) {
                // the dot product takes each pair as built, not an element of
                // pf: the compiler was seen to fold fdot2 over elements of a
                // bit-cast vector into the first element
                const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
                f16x2 h[4];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    h[w] = f16x2{(_Float16)sacc[b][q0 + 2 * w], (_Float16)sacc[b][q0 + 2 * w + 1]};
                    rs[w] = __builtin_amdgcn_fdot2(h[w], ones, rs[w], false);
                }
                pf[2 * b + hsel] = u32x4{__builtin_bit_cast(uint32_t, h[0]), __builtin_bit_cast(uint32_t, h[1]),
                                         __builtin_bit_cast(uint32_t, h[2]), __builtin_bit_cast(uint32_t, h[3])};
            } else {
                pf[2 * b + hsel] = u32x4{pack2<F16>(sacc[b][q0 + 0], sacc[b][q0 + 1]),
                                         pack2<F16>(sacc[b][q0 + 2], sacc[b][q0 + 3]),
                                         pack2<F16>(sacc[b][q0 + 4], sacc[b][q0 + 5]),
                                         pack2<F16>(sacc[b][q0 + 6], sacc[b][q0 + 7])};
            }
        }
    st.l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
}

// O^T += V^T P^T over the tile's 2*NKB 16-key steps.
template <bool F16, int NKB, class VF>
__device__ __forceinline__ void tile_pv(RowState &st, const u32x4 (&pf)[2 * NKB], VF vfrag) {
#pragma unroll
    for (int kk = 0; kk < 2 * NKB; ++kk)
#pragma unroll
        for (int x = 0; x < 4; ++x)
            st.o[x] = mfma32<F16>(vfrag(kk, x), pf[kk], st.o[x]);
}

// S^T of the tile from fp8 K codes (the PAIRED d order of load_q): kpair(b,
// j, f0, f1) widens one 16-byte read of block b's key row into the operands of
// k-steps 2j and 2j+1.  Per block the k-steps still run in ascending order.
template <bool F16, int NKB, class KP>
__device__ __forceinline__ void tile_scores_paired(f32x16 (&sacc)[NKB], const u32x4 (&qf)[8], KP kpair) {
#pragma unroll
    for (int b = 0; b < NKB; ++b)
        sacc[b] = f32x16{};
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u32x4 f[NKB][2];
#pragma unroll
        for (int b = 0; b < NKB; ++b)
            kpair(b, j, f[b][0], f[b][1]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b = 0; b < NKB; ++b)
                sacc[b] = mfma32<F16>(f[b][h], qf[2 * j + h], sacc[b]);
    }
    __builtin_amdgcn_s_setprio(0);
}

template <bool F16, int NKB, bool EXT = false, bool HOIST = false, class KF, class VF>
__device__ __forceinline__ void attend_tile(RowState &st, const u32x4 (&qf)[8], KF kfrag, VF vfrag,
                                            int key0, bool masked, int lim, float c2, int lane,
                                            RowExt ext = RowExt{0, 0, 0.0f}, bool alibi = false) {
    f32x16 sacc[NKB];
    u32x4 pf[2 * NKB];
    tile_scores<F16, NKB, HOIST>(sacc, qf, kfrag);
    tile_softmax<F16, NKB, EXT>(st, sacc, pf, key0, masked, lim, c2, lane, ext, alibi);
    tile_pv<F16, NKB>(st, pf, vfrag);
}

template <bool F16, int NKB, bool EXT = false, class KP, class VF>
__device__ __forceinline__ void attend_tile_paired(RowState &st, const u32x4 (&qf)[8], KP kpair, VF vfrag,
                                                   int key0, bool masked, int lim, float c2, int lane,
                                                   RowExt ext = RowExt{0, 0, 0.0f}, bool alibi = false) {
    f32x16 sacc[NKB];
    u32x4 pf[2 * NKB];
    tile_scores_paired<F16, NKB>(sacc, qf, kpair);
    tile_softmax<F16, NKB, EXT>(st, sacc, pf, key0, masked, lim, c2, lane, ext, alibi);
    tile_pv<F16, NKB>(st, pf, vfrag);
}

// V^T fragment from a row-major [keys][128] LDS V tile with the swz_v layout,
// by two transposing reads.  Lane j of 16-lane group g = lane/16 points at key
// 16kk + 8(g>>1) + 4t + j/4 (t = 0, 1), d 32x + 16(g&1) + 4(j%4) .. +3, and
// receives V[16kk + 8(g>>1) + 4t + e][32x + 16(g&1) + j], e = 0..3.
__device__ __forceinline__ u32x4 vfrag_lds(const uint8_t *sV, int kk, int x, int lane) {
    const int jg = lane & 15;
    const int vrow = 16 * kk + 8 * (lane >> 5) + (jg >> 2);
    const int gran = 4 * x + 2 * ((lane >> 4) & 1) + ((jg & 3) >> 1);
    const uint8_t *va = sV + vrow * 256 + ((gran ^ swz_v(vrow)) << 4) + 8 * (jg & 1);
    const u32x2 w0 = __builtin_bit_cast(u32x2, ds_read_tr16(va));
    const u32x2 w1 = __builtin_bit_cast(u32x2, ds_read_tr16(va + 4 * 256));
    return u32x4{w0[0], w0[1], w1[0], w1[1]};
}

// Row epilogue: normalised output (or split partial) and log-sum-exp of the
// rows of d blocks [x0, x0 + NX).  o holds the blocks' accumulators, m the
// row's reference max, l_row its full weight sum.
template <bool F16, bool SPLIT, int NX>
__device__ __forceinline__ void write_rows(const AttnArgs &a, const f32x16 (&o)[NX], int x0, float m,
                                           float l_row, float v_scale, int64_t tok, int head, int split,
                                           int lane, bool write_lse) {
    const int hl = lane >> 5;
    const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
    const float lse = l_row > 0.0f ? m * kLn2 + __logf(l_row) : neg_inf();
    const float sc = inv * v_scale;
    if constexpr (!SPLIT) {
        uint8_t *op = (uint8_t *)a.out + (tok * a.o_st_tok + (int64_t)head * a.o_st_head) * 2;
#pragma unroll
        for (int x = 0; x < NX; ++x)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * (x0 + x) + 8 * g + 4 * hl;
                const u32x2 w = {pack2<F16>(o[x][4 * g] * sc, o[x][4 * g + 1] * sc),
                                 pack2<F16>(o[x][4 * g + 2] * sc, o[x][4 * g + 3] * sc)};
                *(u32x2 *)(op + d * 2) = w;
            }
        if (write_lse && a.lse_out != nullptr && hl == 0)
            a.lse_out[tok * a.num_q_heads + head] = lse;
    } else {
        const int64_t row = ((int64_t)split * a.num_tokens + tok) * a.num_q_heads + head;
        float *op = a.o_part + row * HD;
#pragma unroll
        for (int x = 0; x < NX; ++x)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * (x0 + x) + 8 * g + 4 * hl;
                *(f32x4 *)(op + d) = f32x4{o[x][4 * g] * sc, o[x][4 * g + 1] * sc,
                                           o[x][4 * g + 2] * sc, o[x][4 * g + 3] * sc};
            }
        if (write_lse && hl == 0)
            a.lse_part[row] = lse;
    }
}

// NaN into a row's output (or split partial) and log-sum-exp: the mark of a
// workgroup whose key-group barrier timed out.  Each lane half writes its own
// d chunks, as write_rows does.
template <bool SPLIT>
__device__ __forceinline__ void poison_row(const AttnArgs &a, int64_t tok, int head, int split, int lane) {
    const int hl = lane >> 5;
    const float nan = __builtin_nanf("");
    if constexpr (!SPLIT) {
        uint8_t *op = (uint8_t *)a.out + (tok * a.o_st_tok + (int64_t)head * a.o_st_head) * 2;
        const uint32_t nan2 = 0x7fff7fffu;      // a NaN in both halves (bf16 and fp16)
#pragma unroll
        for (int g = 0; g < 16; ++g)
            *(u32x2 *)(op + (8 * g + 4 * hl) * 2) = u32x2{nan2, nan2};
        if (a.lse_out != nullptr && hl == 0)
            a.lse_out[tok * a.num_q_heads + head] = nan;
    } else {
        const int64_t row = ((int64_t)split * a.num_tokens + tok) * a.num_q_heads + head;
        float *op = a.o_part + row * HD;
#pragma unroll
        for (int g = 0; g < 16; ++g)
            *(f32x4 *)(op + 8 * g + 4 * hl) = f32x4{nan, nan, nan, nan};
        if (hl == 0)
            a.lse_part[row] = nan;
    }
}

// Q fragments of row (tok, head): B operand of S^T = K Q^T, k-step ks covers
// d 16ks .. 16ks+15 (8 per lane half).  PAIRED (the fp8-cache prefill path):
// k-steps 2j and 2j+1 of lane half h cover d 32j + 16h .. 32j + 16h + 15, so
// one 16-byte read of a key row's codes gives a lane both steps' K operands.
// Zero for rows that do not exist.
template <bool PAIRED = false>
__device__ __forceinline__ void load_q(const AttnArgs &a, u32x4 (&qf)[8], bool row_ok, int64_t tok,
                                       int head, int lane) {
    if (row_ok) {
        const uint8_t *qp = (const uint8_t *)a.q + (tok * a.q_st_tok + (int64_t)head * a.q_st_head) * 2;
        const int hl = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int d0 = PAIRED ? 32 * (ks >> 1) + 16 * hl + 8 * (ks & 1) : 16 * ks + 8 * hl;
            qf[ks] = *(const u32x4 *)(qp + d0 * 2);
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            qf[ks] = u32x4{0, 0, 0, 0};
    }
    // Q is resident before the key loop starts (a wait the compiler tracks, so
    // no later wait is spent on these loads)
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
}

// ------------------------------------------------------------------ prefill kernel

// Query block of prefill workgroup bx and its key-tile range.  The host sizes
// the grid as (T / BLOCK_Q + S) query-block slots per kv head without reading
// device memory; sequence s owns the slots from cu[s] / BLOCK_Q + s, found by
// a binary search over cu_seqlens_q (page "vLLM Triton unified attention
// notes", section kernel_unified_attention_2d: find_seq_idx and the slot
// transform).  False when the slot is empty or the sequence belongs to the
// decode body (uniform over the workgroup).
struct PrefillBlock {
    int kvh, split, s, cu0, q_len, tq0, tq1, kv_len, ctx, kv_end, n_full, first_full, t_begin, t_end;
};

template <bool CAUSAL, bool SPLIT, bool EXT>
__device__ __forceinline__ bool locate_block(const AttnArgs &a, int bx, int split, int TN,
                                             PrefillBlock &B) {
    B.kvh = bx % a.num_kv_heads;
    int slot = bx / a.num_kv_heads;
    if (CAUSAL)
        slot = a.num_qslots - 1 - slot;         // late (long) query blocks first
    B.split = split;
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {                           // largest s with cu[s]/BLOCK_Q + s <= slot
        const int mid = (lo + hi + 1) >> 1;
        if (a.cu_seqlens_q[mid] / a.block_q + mid <= slot)
            lo = mid;
        else
            hi = mid - 1;
    }
    B.s = lo;
    B.cu0 = a.cu_seqlens_q[lo];
    B.q_len = a.cu_seqlens_q[lo + 1] - B.cu0;
    if (a.short_to_decode && B.q_len * a.group <= kDecodeRows)
        return false;                           // the decode body owns this sequence
    B.tq0 = (slot - (B.cu0 / a.block_q + lo)) * a.block_q;
    if (B.tq0 >= B.q_len)
        return false;                           // empty slot
    B.tq1 = min(B.q_len, B.tq0 + a.block_q);
    B.kv_len = a.seqused_k[lo];
    B.ctx = B.kv_len - B.q_len;                 // keys before the first query
    // keys seen by some row / by every row of this block (visibility bounds
    // grow with the row's position, so the first and last token bound them)
    B.kv_end = CAUSAL ? min(B.kv_len, B.ctx + B.tq1) : B.kv_len;
    int full_end = CAUSAL ? min(B.kv_len, B.ctx + B.tq0 + 1) : B.kv_len;
    int kv_begin = 0, full_begin = 0;
    if (EXT) {
        if (a.win_right >= 0) {
            B.kv_end = min(B.kv_end, B.ctx + B.tq1 + a.win_right);
            full_end = min(full_end, B.ctx + B.tq0 + a.win_right + 1);
        }
        if (a.win_left >= 0) {
            kv_begin = max(0, B.ctx + B.tq0 - a.win_left);
            full_begin = max(0, B.ctx + B.tq1 - 1 - a.win_left);
        }
    }
    const int n_tiles = max(B.kv_end, 0) / TN + ((max(B.kv_end, 0) % TN) != 0);
    const int t_first = min(kv_begin / TN, n_tiles);
    B.n_full = max(full_end, 0) / TN;
    B.first_full = full_begin / TN + ((full_begin % TN) != 0);
    B.t_begin = t_first;
    B.t_end = n_tiles;
    if (SPLIT) {
        const int per = (n_tiles - t_first + a.num_splits - 1) / a.num_splits;
        B.t_begin = min(n_tiles, t_first + B.split * per);
        B.t_end = min(n_tiles, B.t_begin + per);
    }
    return true;
}

// Prefill workgroup bx: KG key groups of 4 waves x 32 rows.  Every group
// holds all 128 rows; group g takes the tiles t_begin + g, t_begin + g + KG,
// ... of the block's range through its own two LDS stages, and the groups'
// softmax states are merged at the end (KG = 2 gives two waves per SIMD where
// a launch has only about one workgroup per CU).
template <bool F16, bool FP8KV, bool CAUSAL, bool SPLIT, int KG, bool EXT>
__device__ __forceinline__ void prefill_body(const AttnArgs &a, int bx, int split_ix, int tid_in,
                                             uint8_t *lds) {
    constexpr int NT = 256, TN = 64;
    constexpr int NKB = TN / 32;                // 32-key blocks per tile
    constexpr int KVB = FP8KV ? 1 : 2;          // bytes per cached element
    constexpr int STAGE = 2 * TN * 256;         // bytes of one K + V stage (16-bit in LDS)
    static_assert(KG == 1 || KG == 2, "one or two key groups");
    static_assert(KG * 2 * STAGE + 8 <= lds_bytes(4 * KG) &&
                      (KG == 1 || 4 * kDecodeMergeRows * 64 * 4 <= KG * 2 * STAGE),
                  "stages, counters and merge records fit");

    const int tid = tid_in;
    const int grp = KG == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 8);   // key group
    const int gtid = tid & (NT - 1);            // thread within the group
    const int lane = tid & 63;
    const int wave = gtid >> 6;                 // row wave within the group
    const int hl = lane >> 5;                   // lane half
    const int lc = lane & 31;                   // accumulator column = query row in the wave
    uint8_t *const sK0 = lds + grp * (2 * STAGE);
    uint8_t *const sV0 = sK0 + TN * 256;
    uint8_t *const sK1 = sK0 + STAGE;
    uint8_t *const sV1 = sK1 + TN * 256;
    // key-group barrier counters (one per group), then the lost flag, after
    // both groups' stages
    uint32_t *const gctr = (uint32_t *)(lds + KG * 2 * STAGE) + grp;
    uint32_t *const lost_flag = (uint32_t *)(lds + KG * 2 * STAGE) + 2;
    uint32_t n_sync = 0;
    bool lost = false;                          // a key-group barrier of this wave timed out
    auto loop_sync = [&]() {
        if constexpr (KG == 1)
            __syncthreads();
        else
            lost |= group_barrier(gctr, 4u * ++n_sync, lane, a.spin_limit);
    };

    // ---------------------------------------------------------------- tiler
    PrefillBlock B;
    if (!locate_block<CAUSAL, SPLIT, EXT>(a, bx, split_ix, TN, B))
        return;                                 // uniform, before any barrier
    const int kvh = B.kvh, split = B.split, s = B.s, cu0 = B.cu0;
    const int tq0 = B.tq0, tq1 = B.tq1, kv_len = B.kv_len, ctx = B.ctx, kv_end = B.kv_end;
    const int n_full = B.n_full, first_full = B.first_full, t_begin = B.t_begin, t_end = B.t_end;
    const int G = a.group;
    // iteration k: group g holds tile mine(k) if has(k); barriers follow the
    // iteration count, which is the same for every group
    const int n_it = (t_end - t_begin + KG - 1) / KG;
    auto mine = [&](int k) { return t_begin + grp + KG * k; };
    auto has = [&](int k) { return mine(k) < t_end; };
    if constexpr (KG == 2) {
        if (tid < 3)
            ((uint32_t *)(lds + KG * 2 * STAGE))[tid] = 0;   // ordered by the first full barrier
    }

    // ---------------------------------------------------------------- rows
    const int r = wave * 32 + lc;
    const int tq = r / G;
    const int hg = r - tq * G;
    const int t_loc = tq0 + tq;
    const bool row_ok = t_loc < tq1;            // also false for rows past BLOCK_Q * G
    const int64_t tok = (int64_t)cu0 + t_loc;
    const int head = kvh * G + hg;
    int lim = !row_ok ? 0 : (CAUSAL ? min(kv_len, ctx + t_loc + 1) : kv_len);
    RowExt ext{0, 0, 0.0f};
    const bool alibi = EXT && a.alibi != nullptr;
    if constexpr (EXT) {
        const int pos = ctx + t_loc;
        if (a.win_right >= 0)
            lim = min(lim, pos + a.win_right + 1);
        ext.lo = a.win_left >= 0 ? max(0, pos - a.win_left) : 0;
        ext.pos = pos;
        ext.sl2 = alibi ? a.alibi[head] * kLog2e : 0.0f;
    }
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const bool wave_on = wv * 32 < (tq1 - tq0) * G;       // uniform over the wave
    u32x4 qf[8];
    load_q<FP8KV>(a, qf, row_ok, tok, head, lane);

    // ---------------------------------------------------------------- paging
    const int32_t *btrow = a.block_table + (int64_t)s * a.bt_stride;
    const int lbs = a.log2_block_size;
    const int bs_mask = (1 << lbs) - 1;
    const int last_page = (max(kv_end, 1) - 1) >> lbs;     // later table entries are never read
    const uint8_t *kbase = (const uint8_t *)a.k + (int64_t)kvh * a.kv_st_head * KVB;
    const uint8_t *vbase = (const uint8_t *)a.v + (int64_t)kvh * a.kv_st_head * KVB;

    const float c2 = a.scale_log2 * (FP8KV ? *a.k_scale : 1.0f);   // score -> log2 units
    RowState st;
    init_rows(st);
    // fp8 caches: the tile holds codes (128-byte key rows, 16-byte chunks) and
    // the operands are widened to the q dtype as they are read.  K chunk c of
    // key k sits at position c ^ ((k >> 1) & 7): the 16 lanes of a 16-byte
    // read take 16 different keys (both parities of 8 key pairs) and hit 16
    // distinct 16-byte bank groups.  V chunk c of key k sits at
    // c ^ 2((k >> 1) & 3): the 32 lanes of an 8-bit transposing read take 8
    // consecutive keys x chunks 2x, 2x+1 and hit 32 distinct 8-byte groups.
    auto compute = [&](int tile, const uint8_t *sK, const uint8_t *sV) {
        if constexpr (FP8KV) {
            const int k8swz = (swap23(lc) >> 1) & 7;            // K position XOR of this lane's rows
            const int te = (lane & 15) >> 1, tp = lane & 1;     // transposing-read source row, half
            const int v8swz = 2 * ((te >> 1) & 3);              // V position XOR of key 8h + te
            const int vchunk = (lane >> 4) & 1;                 // chunk 2x + vchunk
            // block b, k-steps 2j, 2j+1: key 32b + swap23(lc), d 32j + 16hl + 0..15
            const uint8_t *krow = sK + swap23(lc) * 128;
            auto kp = [&](int b, int j, u32x4 &f0, u32x4 &f1) {
                const u32x4 w = *(const u32x4 *)(krow + 32 * b * 128 + (((2 * j + hl) ^ k8swz) << 4));
                f0 = widen_fp8<F16>(u32x2{w[0], w[1]});
                f1 = widen_fp8<F16>(u32x2{w[2], w[3]});
            };
            // V^T operand of 16-key step kk, d block x: lane (h, lc) receives
            // keys 16kk + 8h + 0..7 at d 32x + lc (byte e = key 16kk + 8h + e)
            const uint8_t *vrow = sV + (8 * hl + te) * 128 + 8 * tp;
            auto vf = [&](int kk, int x) {
                const uint8_t *src = vrow + kk * 16 * 128 + ((((2 * x) ^ v8swz) + vchunk) << 4);
                const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) i32x2 *)(src));
                return widen_fp8<F16>(u32x2{(uint32_t)w[0], (uint32_t)w[1]});
            };
            attend_tile_paired<F16, NKB, EXT>(st, qf, kp, vf, tile * TN,
                                              tile >= n_full || (EXT && tile < first_full), lim, c2,
                                              lane, ext, alibi);
        } else {
            const uint8_t *krow = sK + swap23(lc) * 256;
            auto kf = [&](int b, int ks) {
                return *(const u32x4 *)(krow + 32 * b * 256 + (((2 * ks + hl) ^ (lane & 15)) << 4));
            };
            auto vf = [&](int kk, int x) { return vfrag_lds(sV, kk, x, lane); };
            // the K fragments are read ahead of the score chain where that
            // measured faster and the register file has room: fp16, one key
            // group, no window or ALiBi (bf16 mixed batches and the ALiBi
            // path measured about 1 % slower with it)
            constexpr bool hoist = F16 && KG == 1 && !EXT;
            attend_tile<F16, NKB, EXT, hoist>(st, qf, kf, vf, tile * TN,
                                              tile >= n_full || (EXT && tile < first_full), lim, c2,
                                              lane, ext, alibi);
        }
    };

    {
        // K/V go straight from HBM into LDS (global_load_lds, 16 bytes per
        // lane), no register staging; fp8 caches stay codes in LDS (widened
        // as the operands are read).  Wave w fills keys 16w .. 16w+15 of the
        // tile (one page: a page holds >= 16 keys): 16-bit rows with four
        // 4-key instructions per tensor, fp8 rows with two 8-key
        // instructions.  Lane l of an instruction lands at LDS byte 16*l of
        // its rows, so it fetches the chunk whose swizzled position that is.
        // The DMA of tile + 1 runs under the compute of tile; one barrier per
        // tile.  The page id is a scalar load fetched a tile ahead.
        constexpr int RB = 128 * KVB;                     // bytes of a key row in LDS
        constexpr int NI = FP8KV ? 2 : 4;                 // instructions per tensor and tile
        constexpr int RPI = 16 / NI;                      // key rows per instruction
        constexpr int CPR = RB / 16;                      // 16-byte chunks per row
        // per-lane global offsets of the instructions (the row group
        // included, so all share the page's scalar base); m0 of each
        // instruction is the wave's first row in the group's LDS area plus a
        // compile-time offset
        const int lrow = FP8KV ? lane >> 3 : lane >> 4;  // row within an instruction's group
        const int pc = lane & (CPR - 1);                  // chunk position within the row
        uint32_t koff[NI], voff[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t rofs = (uint32_t)((RPI * i + lrow) * a.kv_st_slot * KVB);
            if constexpr (FP8KV) {
                const int kl = RPI * i + lrow;            // key within the wave's 16 (same bits 1..3)
                koff[i] = rofs + (uint32_t)((pc ^ ((kl >> 1) & 7)) << 4);
                voff[i] = rofs + (uint32_t)((pc ^ (2 * ((kl >> 1) & 3))) << 4);
            } else {
                koff[i] = rofs + (uint32_t)((pc ^ swz_k(RPI * i + lrow)) << 4);
                voff[i] = rofs + (uint32_t)((pc ^ swz_v(lrow)) << 4);
            }
        }
        const int wrow = 16 * wv;                         // this wave's first key in the tile
        const uint32_t lds_row0 = (uint32_t)reinterpret_cast<uintptr_t>(
            (__attribute__((address_space(3))) uint8_t *)(sK0)) + (uint32_t)(wrow * RB);
        int32_t blk = 0;
        auto fetch_id = [&](int tile) {
            blk = sload(btrow + min((tile * TN + wrow) >> lbs, last_page));
        };
        // STG: 0 fills the first K/V stage of the group, 1 the second
        auto dma_tile = [&](int tile, auto stg) {
            constexpr int KOFS = decltype(stg)::value * STAGE, VOFS = KOFS + TN * 256;
            const int j = tile * TN + wrow;
            const int64_t pofs =
                ((int64_t)blk * a.kv_st_blk + (int64_t)(j & bs_mask) * a.kv_st_slot) * KVB;
            const uint8_t *gk = kbase + pofs, *gv = vbase + pofs;
            lds_dma16_at<KOFS + 0 * RPI * RB>(gk, koff[0], lds_row0);
            lds_dma16_at<VOFS + 0 * RPI * RB>(gv, voff[0], lds_row0);
            lds_dma16_at<KOFS + 1 * RPI * RB>(gk, koff[1], lds_row0);
            lds_dma16_at<VOFS + 1 * RPI * RB>(gv, voff[1], lds_row0);
            if constexpr (NI == 4) {
                lds_dma16_at<KOFS + 2 * RPI * RB>(gk, koff[2], lds_row0);
                lds_dma16_at<VOFS + 2 * RPI * RB>(gv, voff[2], lds_row0);
                lds_dma16_at<KOFS + 3 * RPI * RB>(gk, koff[3], lds_row0);
                lds_dma16_at<VOFS + 3 * RPI * RB>(gv, voff[3], lds_row0);
            }
        };
        using Stg0 = std::integral_constant<int, 0>;
        using Stg1 = std::integral_constant<int, 1>;
        // keys at or past kv_end came from a clamped (allocated) page: zero
        // their V rows so that weight 0 times whatever was there stays 0
        // (their scores are masked)
        auto zero_tail = [&](int tile, uint8_t *sV) {
            if ((tile + 1) * TN > kv_end) {
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    if (tile * TN + wrow + RPI * i + lrow >= kv_end)
                        *(u32x4 *)(sV + (wrow + RPI * i) * RB + 16 * lane) = u32x4{0, 0, 0, 0};
            }
        };
        if (n_it > 0) {
            if (has(0)) {
                fetch_id(mine(0));
                dma_tile(mine(0), Stg0{});
                if (has(1))
                    fetch_id(mine(1));
            }
            wait_vmem();
            if (has(0))
                zero_tail(mine(0), sV0);
            __syncthreads();
        }
        // unrolled by two so that each stage's LDS addresses are constants
        auto step = [&](int k, uint8_t *cK, uint8_t *cV, auto nstg, uint8_t *nV) {
            if (has(k + 1)) {
                dma_tile(mine(k + 1), nstg);
                if (has(k + 2))
                    fetch_id(mine(k + 2));
            }
            if (wave_on && has(k))
                compute(mine(k), cK, cV);
            if (k + 1 < n_it) {
                wait_vmem();
                if (has(k + 1))
                    zero_tail(mine(k + 1), nV);
                loop_sync();
            }
        };
        for (int k = 0; k < n_it; k += 2) {
            step(k, sK0, sV0, Stg1{}, sV1);
            if (k + 1 < n_it)
                step(k + 1, sK1, sV1, Stg0{}, sV0);
        }
    }
    // ---------------------------------------------------------------- epilogue
    if constexpr (KG == 1) {
        if (!wave_on)
            return;
        const float l_row = xhalf_sum(st.l);
        if (!row_ok)
            return;
        write_rows<F16, SPLIT, 4>(a, st.o, 0, st.m, l_row, FP8KV ? *a.v_scale : 1.0f, tok, head,
                                  split, lane, true);
    } else {
        // group 1 leaves (o, m, l) per lane in LDS; group 0 merges them into
        // its own state (both hold the same rows in the same lanes)
        const float l_row = xhalf_sum(st.l);
        mark_lost(lost_flag, lost, lane);
        __syncthreads();                        // both groups are done with their stages
        const bool wg_lost = __hip_atomic_load(lost_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
        float *rec = (float *)lds + wave * (kDecodeMergeRows * 64);
        if (grp == 1) {
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    rec[(16 * x + i) * 64 + lane] = st.o[x][i];
            rec[64 * 64 + lane] = st.m;
            rec[65 * 64 + lane] = l_row;
        }
        __syncthreads();
        if (grp == 1 || !wave_on)
            return;
        const float m1 = rec[64 * 64 + lane];
        const float M = fmaxf(st.m, m1);
        const float s0 = (st.m == neg_inf()) ? 0.0f : __builtin_amdgcn_exp2f(st.m - M);
        const float s1 = (m1 == neg_inf()) ? 0.0f : __builtin_amdgcn_exp2f(m1 - M);
        const float L = s0 * l_row + s1 * rec[65 * 64 + lane];
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                st.o[x][i] = s0 * st.o[x][i] + s1 * rec[(16 * x + i) * 64 + lane];
        if (!row_ok)
            return;
        if (wg_lost) {
            poison_row<SPLIT>(a, tok, head, split, lane);
            return;
        }
        write_rows<F16, SPLIT, 4>(a, st.o, 0, M, L, FP8KV ? *a.v_scale : 1.0f, tok, head, split,
                                  lane, true);
    }
}

// ------------------------------------------------------------------ fp8-MFMA prefill

// Opt-in fp8 compute for fp8 caches (the fp8 attention variants of page
// "flashatten takeaways EP2 工程", section "源代码接口", and the FA3 fp8 path of
// page "Fused Attention"): each query row is quantised to e4m3 with its own
// scale amax / 448, K and V stay e4m3 from HBM through LDS to the matrix
// cores, S^T = K Q^T and O^T = V^T P^T run as 32x32x64 fp8 MFMAs, and P is
// rounded to e4m3 (weights are <= 2^8 < 448 under the lazy rescale).  The row
// sum adds the fp32 weights before rounding, as the bf16 path does.
//
// LDS layouts of a 64-key tile (128-byte rows of codes, 16-byte chunks):
//   K: chunk c of key k at c ^ gk(k), gk = ((k >> 1) & 3) | (((k >> 4) & 1) << 2);
//   V: chunk c of key k at c ^ 2((k >> 1) & 3), so the 32 lanes of an 8-bit
//      transposing read (8 consecutive keys x chunks 2x, 2x+1) hit 32
//      distinct 8-byte bank groups.
// MFMA row i of a 32-key score block reads key pk(i) = 16((i >> 2) & 1) +
// 4(i >> 3) + (i & 3), which puts keys 16h .. 16h+15 of the block in
// accumulator registers 0..15 of lane half h: the 32 weights a lane holds are
// the bytes of its P^T operand, and the V^T operand gathers the same keys with
// four 8-bit transposing reads.
__device__ __forceinline__ int gk_swz(int k) { return ((k >> 1) & 3) | (((k >> 4) & 1) << 2); }
__device__ __forceinline__ int gv_swz(int k) { return 2 * ((k >> 1) & 3); }
__device__ __forceinline__ int pk_row(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

template <bool F16, bool CAUSAL, bool SPLIT, int KG>
__device__ __forceinline__ void prefill_body_f8(const AttnArgs &a, int bx, int split_ix, int tid_in,
                                                uint8_t *lds) {
    constexpr int NT = 256, TN = 64;
    constexpr int TB = TN * 128;                // bytes of one K (or V) tile of codes
    constexpr int STAGE = 2 * TB;
    static_assert(KG == 1 || KG == 2, "one or two key groups");

    const int tid = tid_in;
    const int grp = KG == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 8);
    const int gtid = tid & (NT - 1);
    const int lane = tid & 63;
    const int wave = gtid >> 6;
    const int hl = lane >> 5;
    const int lc = lane & 31;
    uint8_t *const sK0 = lds + grp * (2 * STAGE);
    uint8_t *const sV0 = sK0 + TB;
    uint8_t *const sK1 = sK0 + STAGE;
    uint8_t *const sV1 = sK1 + TB;
    // key-group barrier counters and the lost flag (the same place as the
    // 16-bit body's)
    uint32_t *const gctr = (uint32_t *)(lds + KG * 2 * (2 * TN * 256)) + grp;
    uint32_t *const lost_flag = (uint32_t *)(lds + KG * 2 * (2 * TN * 256)) + 2;
    uint32_t n_sync = 0;
    bool lost = false;
    auto loop_sync = [&]() {
        if constexpr (KG == 1)
            __syncthreads();
        else
            lost |= group_barrier(gctr, 4u * ++n_sync, lane, a.spin_limit);
    };

    PrefillBlock B;
    if (!locate_block<CAUSAL, SPLIT, false>(a, bx, split_ix, TN, B))
        return;
    const int kvh = B.kvh, split = B.split, s = B.s, cu0 = B.cu0;
    const int tq0 = B.tq0, tq1 = B.tq1, kv_len = B.kv_len, ctx = B.ctx, kv_end = B.kv_end;
    const int n_full = B.n_full, t_begin = B.t_begin, t_end = B.t_end;
    const int G = a.group;
    const int n_it = (t_end - t_begin + KG - 1) / KG;
    auto mine = [&](int k) { return t_begin + grp + KG * k; };
    auto has = [&](int k) { return mine(k) < t_end; };
    if constexpr (KG == 2) {
        if (tid < 3)
            ((uint32_t *)(lds + KG * 2 * (2 * TN * 256)))[tid] = 0;
    }

    const int r = wave * 32 + lc;
    const int tq = r / G;
    const int hg = r - tq * G;
    const int t_loc = tq0 + tq;
    const bool row_ok = t_loc < tq1;
    const int64_t tok = (int64_t)cu0 + t_loc;
    const int head = kvh * G + hg;
    const int lim = !row_ok ? 0 : (CAUSAL ? min(kv_len, ctx + t_loc + 1) : kv_len);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const bool wave_on = wv * 32 < (tq1 - tq0) * G;

    // Q row -> e4m3 codes: lane half hl holds d = 64 st + 32 hl + b (b < 32)
    // of k-step st as B-operand bytes b
    i32x8 qc[2];
    float sq = 1.0f;
    {
        float qv[64];
        if (row_ok) {
            const uint8_t *qp = (const uint8_t *)a.q + (tok * a.q_st_tok + (int64_t)head * a.q_st_head) * 2;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x4 w = *(const u32x4 *)(qp + (64 * st + 32 * hl + 8 * c) * 2);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float lo, hi;
                        if constexpr (F16) {
                            // halves taken as scalars (element access on a
                            // bit-cast f16x2 was seen to be folded wrongly)
                            lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] & 0xffffu));
                            hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] >> 16));
                        } else {
                            lo = __uint_as_float(w[e] << 16);
                            hi = __uint_as_float(w[e] & 0xffff0000u);
                        }
                        qv[32 * st + 8 * c + 2 * e] = lo;
                        qv[32 * st + 8 * c + 2 * e + 1] = hi;
                    }
                }
        } else {
#pragma unroll
            for (int i = 0; i < 64; ++i)
                qv[i] = 0.0f;
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 64; ++i)
            amax = fmaxf(amax, __builtin_fabsf(qv[i]));
        amax = xhalf_max(amax);
        sq = amax > 0.0f ? amax / 448.0f : 1.0f;        // IEEE division (the code decision)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    x[e] = fminf(fmaxf(qv[32 * st + 4 * w + e] / sq, -448.0f), 448.0f);
                qc[st][w] = (int)pack_fp8x4(x[0], x[1], x[2], x[3]);
            }
    }

    const int32_t *btrow = a.block_table + (int64_t)s * a.bt_stride;
    const int lbs = a.log2_block_size;
    const int bs_mask = (1 << lbs) - 1;
    const int last_page = (max(kv_end, 1) - 1) >> lbs;
    const uint8_t *kbase = (const uint8_t *)a.k + (int64_t)kvh * a.kv_st_head;
    const uint8_t *vbase = (const uint8_t *)a.v + (int64_t)kvh * a.kv_st_head;
    const float c2 = a.scale_log2 * *a.k_scale * sq;  // code product -> log2 units

    RowState st;
    init_rows(st);

    // direct loads: wave w fills keys 16w .. 16w+15 of the tile (one page)
    // with two 8-key instructions per tensor; lane l lands at LDS byte 16 l of
    // the instruction's 8 rows (row l / 8, chunk position l % 8) and fetches
    // the chunk the swizzle puts there
    const int lrow = lane >> 3, pc = lane & 7;
    const int wrow = 16 * wv;
    uint32_t koff[2], voff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int kl = wrow + 8 * i + lrow;
        koff[i] = (uint32_t)(lrow * a.kv_st_slot + 16 * (pc ^ gk_swz(kl)));
        voff[i] = (uint32_t)(lrow * a.kv_st_slot + 16 * (pc ^ gv_swz(kl)));
    }
    int32_t blk = 0;
    auto fetch_id = [&](int tile) { blk = sload(btrow + min((tile * TN + wrow) >> lbs, last_page)); };
    auto dma_tile = [&](int tile, uint8_t *sK, uint8_t *sV) {
        const int j = tile * TN + wrow;
        const int64_t pofs = (int64_t)blk * a.kv_st_blk + (int64_t)(j & bs_mask) * a.kv_st_slot;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int64_t gofs = pofs + (int64_t)(8 * i) * a.kv_st_slot;
            lds_dma16(kbase + gofs, koff[i], sK + (wrow + 8 * i) * 128);
            lds_dma16(vbase + gofs, voff[i], sV + (wrow + 8 * i) * 128);
        }
    };
    // keys at or past kv_end came from a clamped page: zero their V rows
    auto zero_tail = [&](int tile, uint8_t *sV) {
        if ((tile + 1) * TN > kv_end) {
            const int row = wrow + (lane >> 2);
            if (tile * TN + row >= kv_end) {
                u32x4 *dst = (u32x4 *)(sV + row * 128 + 32 * (lane & 3));
                dst[0] = u32x4{0, 0, 0, 0};
                dst[1] = u32x4{0, 0, 0, 0};
            }
        }
    };

    // per-lane constants of the operand reads
    const int krow0 = pk_row(lc);
    const int g4 = lane >> 4;                   // 16-lane group of the transposing reads
    const int te = (lane & 15) >> 1, tp = lane & 1;
    auto compute = [&](int tile, const uint8_t *sK, const uint8_t *sV) {
        f32x16 sacc[2];
        sacc[0] = f32x16{};
        sacc[1] = f32x16{};
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int stp = 0; stp < 2; ++stp)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int kr = krow0 + 32 * b;
                const int c0 = 4 * stp + 2 * hl;
                const u32x4 lo = *(const u32x4 *)(sK + kr * 128 + ((c0 ^ gk_swz(kr)) << 4));
                const u32x4 hi = *(const u32x4 *)(sK + kr * 128 + (((c0 + 1) ^ gk_swz(kr)) << 4));
                const i32x8 av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                sacc[b] = mfma32_f8(av, qc[stp], sacc[b]);
            }
        __builtin_amdgcn_s_setprio(0);

        // mask (register q of block b holds key 32 b + 16 hl + q), max, lazy
        // rescale, weights
        const int key0 = tile * TN;
        if (tile >= n_full) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    if (key0 + 32 * b + 16 * hl + q >= lim)
                        sacc[b][q] = neg_inf();
        }
        float mx = neg_inf();
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int q = 0; q < 16; ++q)
                mx = fmaxf(mx, sacc[b][q]);
        mx = xhalf_max(mx);
        const float tmax = mx * c2;
        const bool grow = tmax > st.m + kRescaleLog2;
        if (__ballot(grow) != 0) {
            const float alpha = grow ? __builtin_amdgcn_exp2f(st.m - tmax) : 1.0f;
            st.m = grow ? tmax : st.m;
            st.l *= alpha;
#pragma unroll
            for (int x = 0; x < 4; ++x)
                st.o[x] *= alpha;
        }
        const float m_use = (st.m == neg_inf()) ? 0.0f : st.m;
        float rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const float pw = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[b][q], c2, -m_use));
                sacc[b][q] = pw;
                rs[q & 3] += pw;
            }
        st.l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
        // P^T operand: byte 16 b + q = register q of block b
        i32x8 pf;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int b = w >> 2, q0 = 4 * (w & 3);
            pf[w] = (int)pack_fp8x4(sacc[b][q0], sacc[b][q0 + 1], sacc[b][q0 + 2], sacc[b][q0 + 3]);
        }

        // O^T += V^T P^T over the 4 d blocks; V^T bytes 8 o + e of lane half
        // h are key 16 h + 8 (o & 1) + 32 (o >> 1) + e at d = 32 x + lane % 32
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            i32x8 av;
#pragma unroll
            for (int o = 0; o < 4; ++o) {
                const int key = 16 * hl + 8 * (o & 1) + 32 * (o >> 1) + te;
                const int c = 2 * x + (g4 & 1);
                const uint8_t *src = sV + key * 128 + ((c ^ gv_swz(key)) << 4) + 8 * tp;
                const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) i32x2 *)(src));
                av[2 * o] = w[0];
                av[2 * o + 1] = w[1];
            }
            st.o[x] = mfma32_f8(av, pf, st.o[x]);
        }
    };

    if (n_it > 0) {
        if (has(0)) {
            fetch_id(mine(0));
            dma_tile(mine(0), sK0, sV0);
            if (has(1))
                fetch_id(mine(1));
        }
        wait_vmem();
        if (has(0))
            zero_tail(mine(0), sV0);
        __syncthreads();
    }
    auto step = [&](int k, uint8_t *cK, uint8_t *cV, uint8_t *nK, uint8_t *nV) {
        if (has(k + 1)) {
            dma_tile(mine(k + 1), nK, nV);
            if (has(k + 2))
                fetch_id(mine(k + 2));
        }
        if (wave_on && has(k))
            compute(mine(k), cK, cV);
        if (k + 1 < n_it) {
            wait_vmem();
            if (has(k + 1))
                zero_tail(mine(k + 1), nV);
            loop_sync();
        }
    };
    for (int k = 0; k < n_it; k += 2) {
        step(k, sK0, sV0, sK1, sV1);
        if (k + 1 < n_it)
            step(k + 1, sK1, sV1, sK0, sV0);
    }

    // epilogue (o holds V codes x rounded weights; v_scale / l normalises)
    if constexpr (KG == 1) {
        if (!wave_on)
            return;
        const float l_row = xhalf_sum(st.l);
        if (!row_ok)
            return;
        write_rows<F16, SPLIT, 4>(a, st.o, 0, st.m, l_row, *a.v_scale, tok, head, split, lane, true);
    } else {
        const float l_row = xhalf_sum(st.l);
        mark_lost(lost_flag, lost, lane);
        __syncthreads();
        const bool wg_lost = __hip_atomic_load(lost_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
        float *rec = (float *)lds + wave * (kDecodeMergeRows * 64);
        if (grp == 1) {
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    rec[(16 * x + i) * 64 + lane] = st.o[x][i];
            rec[64 * 64 + lane] = st.m;
            rec[65 * 64 + lane] = l_row;
        }
        __syncthreads();
        if (grp == 1 || !wave_on)
            return;
        const float m1 = rec[64 * 64 + lane];
        const float M = fmaxf(st.m, m1);
        const float s0 = (st.m == neg_inf()) ? 0.0f : __builtin_amdgcn_exp2f(st.m - M);
        const float s1 = (m1 == neg_inf()) ? 0.0f : __builtin_amdgcn_exp2f(m1 - M);
        const float L = s0 * l_row + s1 * rec[65 * 64 + lane];
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                st.o[x][i] = s0 * st.o[x][i] + s1 * rec[(16 * x + i) * 64 + lane];
        if (!row_ok)
            return;
        if (wg_lost) {
            poison_row<SPLIT>(a, tok, head, split, lane);
            return;
        }
        write_rows<F16, SPLIT, 4>(a, st.o, 0, M, L, *a.v_scale, tok, head, split, lane, true);
    }
}

// ------------------------------------------------------------------ decode kernel

// Sequences with q_len * G <= 32 rows.  Grid (S * Hkv, splits).  The NW waves
// of a workgroup hold the same rows and take the key units u0 + w, u0 + w + NW,
// ... of the split's range; a unit is 32 keys.  Per unit, K and V rows are
// loaded whole (coalesced, one unit ahead) into registers, then written into
// the wave's own LDS stages, from which the score fragments are read like the
// prefill body's (K) and the V^T fragments with transposing reads.  (Loading
// K straight in the MFMA operand layout would make every load instruction
// touch 32 key rows; whole-row loads stream about 7% faster.)  The loads of
// unit u + NW are in flight while unit u is computed; no barrier until the
// final merge of the waves' softmax states.
template <bool F16, bool FP8KV, bool CAUSAL, bool SPLIT, int NW, bool EXT>
__device__ __forceinline__ void decode_body(const AttnArgs &a, int bx, int split, int tid_in,
                                            uint8_t *lds) {
    constexpr int NKB = 1;                      // 32-key blocks per unit
    constexpr int UK = 32 * NKB;                // keys per unit
    constexpr int KVB = FP8KV ? 1 : 2;
    constexpr int VST = UK * 256;               // bytes of a wave's V stage (16-bit in LDS)
    constexpr int MROWS = kDecodeMergeRows;
    static_assert(NW * 2 * VST <= lds_bytes(NW) && NW * MROWS * 64 * 4 <= lds_bytes(NW), "LDS budget");

    const int tid = tid_in;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hl = lane >> 5;
    const int lc = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(wave);

    const int s = bx / a.num_kv_heads;
    const int kvh = bx - s * a.num_kv_heads;
    const int cu0 = a.cu_seqlens_q[s];
    const int q_len = a.cu_seqlens_q[s + 1] - cu0;
    const int G = a.group;
    if (q_len == 0 || q_len * G > kDecodeRows)
        return;                                 // empty, or owned by the prefill kernel
    const int kv_len = a.seqused_k[s];
    const int ctx = kv_len - q_len;
    int kv_end = CAUSAL ? min(kv_len, ctx + q_len) : kv_len;
    int full_end = CAUSAL ? min(kv_len, ctx + 1) : kv_len;
    int kv_begin = 0, full_begin = 0;
    if (EXT) {
        if (a.win_right >= 0) {
            kv_end = min(kv_end, ctx + q_len + a.win_right);
            full_end = min(full_end, ctx + a.win_right + 1);
        }
        if (a.win_left >= 0) {
            kv_begin = max(0, ctx - a.win_left);
            full_begin = max(0, ctx + q_len - 1 - a.win_left);
        }
    }
    const int n_units = max(kv_end, 0) / UK + ((max(kv_end, 0) % UK) != 0);
    const int u_first = min(kv_begin / UK, n_units);
    const int n_full = max(full_end, 0) / UK;
    const int first_full = full_begin / UK + ((full_begin % UK) != 0);
    int u_begin = u_first, u_end = n_units;
    if (SPLIT) {
        const int per = (n_units - u_first + a.num_splits - 1) / a.num_splits;
        u_begin = min(n_units, u_first + split * per);
        u_end = min(n_units, u_begin + per);
    }

    // rows (the same in every wave)
    const int tq = lc / G;
    const int hg = lc - tq * G;
    const bool row_ok = tq < q_len;
    const int64_t tok = (int64_t)cu0 + tq;
    const int head = kvh * G + hg;
    int lim = !row_ok ? 0 : (CAUSAL ? min(kv_len, ctx + tq + 1) : kv_len);
    RowExt ext{0, 0, 0.0f};
    const bool alibi = EXT && a.alibi != nullptr;
    if constexpr (EXT) {
        const int pos = ctx + tq;
        if (a.win_right >= 0)
            lim = min(lim, pos + a.win_right + 1);
        ext.lo = a.win_left >= 0 ? max(0, pos - a.win_left) : 0;
        ext.pos = pos;
        ext.sl2 = alibi && head < a.num_q_heads ? a.alibi[head] * kLog2e : 0.0f;
    }

    // paging: a unit's keys lie in at most two pages (keys 0-15 and 16-31 of
    // the unit, a page holding >= 16 keys); their ids are scalar loads fetched
    // one unit ahead of the K/V loads that use them
    static_assert(NKB == 1, "one 32-key block per unit");
    const int32_t *btrow = a.block_table + (int64_t)s * a.bt_stride;
    const int lbs = a.log2_block_size;
    const int bs_mask = (1 << lbs) - 1;
    const int last_page = (max(kv_end, 1) - 1) >> lbs;
    const uint8_t *kbase = (const uint8_t *)a.k + (int64_t)kvh * a.kv_st_head * KVB;
    const uint8_t *vbase = (const uint8_t *)a.v + (int64_t)kvh * a.kv_st_head * KVB;
    int32_t ids[2];
    auto fetch_ids = [&](int u) {
        ids[0] = sload(btrow + min((u * UK) >> lbs, last_page));
        ids[1] = sload(btrow + min((u * UK + 16) >> lbs, last_page));
    };

    // K and V: instruction i covers keys 4i .. 4i+3 of the unit, 16 lanes
    // per key row (16 bytes of a 16-bit row, 8 codes of an fp8 row).  One
    // page per instruction, whole rows per instruction (coalesced).  Both go
    // through the wave's own LDS stages (K with the swz_k layout the score
    // fragments are read from, V with swz_v), lane l writing granule l % 16
    // of its row (an fp8 lane's 8 codes widen to one granule), so each
    // 16-lane store pass covers the 16 positions of one row.
    constexpr int VKI = 4;                      // keys per instruction
    constexpr int VNI = UK / VKI;               // instructions per unit
    const int vkey = lane >> 4;
    const int vch = lane & 15;                  // granule of the row (16-bit)
    const uint32_t vlofs = (uint32_t)(vkey * a.kv_st_slot * KVB + 16 * KVB / 2 * vch);
    // units in flight per wave: two for fp8 caches (their register sets are
    // half as large), one for 16-bit caches (a second set would spill)
    constexpr int NSET = FP8KV ? 2 : 1;
    using LT = std::conditional_t<FP8KV, u32x2, u32x4>;   // one lane's share of a row
    LT kr[NSET][VNI], vr[NSET][VNI];
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, NSET - 1>;
    auto load_kv = [&](int u, auto set) {
        constexpr int SI = decltype(set)::value;
#pragma unroll
        for (int i = 0; i < VNI; ++i) {
            const int jb = u * UK + VKI * i;
            const int64_t pofs = ((int64_t)(VKI * i < 16 ? ids[0] : ids[1]) * a.kv_st_blk +
                                  (int64_t)(jb & bs_mask) * a.kv_st_slot) * KVB;
            // streamed once: non-temporal, so the stream does not evict
            // what other workgroups reuse from the L2
            kr[SI][i] = __builtin_nontemporal_load((const LT *)(kbase + pofs + vlofs));
            vr[SI][i] = __builtin_nontemporal_load((const LT *)(vbase + pofs + vlofs));
        }
    };
    uint8_t *const sK = lds + wv * (2 * VST);
    uint8_t *const sV = sK + VST;
    auto store_kv = [&](int u, auto set) {
        constexpr int SI = decltype(set)::value;
        const bool full = (u + 1) * UK <= kv_end;
#pragma unroll
        for (int i = 0; i < VNI; ++i) {
            const int row = VKI * i + vkey;
            u32x4 k, v;
            if constexpr (FP8KV) {
                k = widen_fp8<F16>(kr[SI][i]);  // 8 codes = d 8vch .. 8vch+7 = granule vch
                v = widen_fp8<F16>(vr[SI][i]);
            } else {
                k = kr[SI][i];
                v = vr[SI][i];
            }
            if (!full && u * UK + row >= kv_end)
                v = u32x4{0, 0, 0, 0};          // clamped-page keys weigh 0; zero their values
            *(u32x4 *)(sK + row * 256 + ((vch ^ swz_k(row)) << 4)) = k;
            *(u32x4 *)(sV + row * 256 + ((vch ^ swz_v(row)) << 4)) = v;
        }
    };

    RowState st;
    init_rows(st);
    u32x4 qf[8];
    const float c2 = a.scale_log2 * (FP8KV ? *a.k_scale : 1.0f);
    const uint8_t *krow = sK + swap23(lc) * 256;
    auto step = [&](int u, auto set) {
        store_kv(u, set);                       // K, V(u) registers -> this wave's stages
        if (u + NSET * NW < u_end) {            // ids of that unit were fetched last step
            load_kv(u + NSET * NW, set);
            if (u + (NSET + 1) * NW < u_end)
                fetch_ids(u + (NSET + 1) * NW);
        }
        auto kf = [&](int b, int ks) {
            return *(const u32x4 *)(krow + 32 * b * 256 + (((2 * ks + hl) ^ (lane & 15)) << 4));
        };
        auto vf = [&](int kk, int x) { return vfrag_lds(sV, kk, x, lane); };
        attend_tile<F16, NKB, EXT>(st, qf, kf, vf, u * UK, u >= n_full || (EXT && u < first_full), lim, c2,
                                   lane, ext, alibi);
    };
    // first unit's loads go out before Q's
    int u = u_begin + wv;
    if (u < u_end) {
        fetch_ids(u);
        load_kv(u, S0{});
        if constexpr (NSET == 2) {
            if (u + NW < u_end) {
                fetch_ids(u + NW);
                load_kv(u + NW, S1{});
            }
        }
        if (u + NSET * NW < u_end)
            fetch_ids(u + NSET * NW);
    }
    load_q(a, qf, row_ok, tok, head, lane);
    for (; u < u_end; u += NSET * NW) {
        step(u, S0{});
        if constexpr (NSET == 2) {
            if (u + NW < u_end)
                step(u + NW, S1{});
        }
    }

    // merge the waves' states: each wave writes (o, m, l) per lane, then wave
    // w < 4 combines d block w of every row and writes it
    const float l_row = xhalf_sum(st.l);
    __syncthreads();                            // every wave is done with its V stage
    float *mrec = (float *)lds + wv * (MROWS * 64);
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            mrec[(16 * x + i) * 64 + lane] = st.o[x][i];
    mrec[64 * 64 + lane] = st.m;
    mrec[65 * 64 + lane] = l_row;
    __syncthreads();
    if (wv >= 4)
        return;
    const float *mall = (const float *)lds;
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < NW; ++w)
        M = fmaxf(M, mall[w * MROWS * 64 + 64 * 64 + lane]);
    float L = 0.0f;
    f32x16 ob[1];
    ob[0] = f32x16{};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float mw = mall[w * MROWS * 64 + 64 * 64 + lane];
        const float sw = (mw == neg_inf()) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
        L += sw * mall[w * MROWS * 64 + 65 * 64 + lane];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            ob[0][i] += sw * mall[w * MROWS * 64 + (16 * wv + i) * 64 + lane];
    }
    if (!row_ok)
        return;
    write_rows<F16, SPLIT, 1>(a, ob, wv, M, L, FP8KV ? *a.v_scale : 1.0f, tok, head, split, lane,
                              wv == 0);
}

// ------------------------------------------------------------------ the kernel

// One launch for both paths: workgroups [0, decode_wgs) run the decode body,
// the rest the prefill body.  Decode workgroups come first so that, in a
// mixed batch, their memory-bound streaming shares the CUs with the
// compute-bound prefill workgroups from the start instead of trailing them.
// KG = 1: two 4-wave workgroups per CU whose waves pair up on each SIMD (wave
// w of both on SIMD w), so the softmax of one wave overlaps the MFMAs of the
// other.  KG = 2 (split launches with prefill work, which have few query
// blocks per kv head): one 8-wave workgroup per CU, the prefill body's two key
// groups (or 8 decode waves) filling the same two slots per SIMD.
// EXT: the local-window / ALiBi path (a separate instantiation, so the plain
// path carries none of its per-element work).
// F8MM (fp8 caches only, without EXT): the prefill rows use the fp8-MFMA
// body; decode rows keep the 16-bit path.
//
// MIX (unsplit prefill, split decode rows: a batch that mixes both kinds of
// sequence): the decode rows' key ranges are split num_splits ways into
// partials that a decode-row combine merges, while prefill workgroups write
// their rows directly.  The grid is one-dimensional in blocks of 8 positions
// (a position's XCD is its index mod 8, so every item keeps the XCD of its
// index and the query blocks of one kv head keep sharing an L2); the
// mix_dblocks decode blocks are spread evenly over the first mix_region
// blocks (the first half of the grid), so that the short split decode
// workgroups stream alongside the prefill ones instead of taking every slot
// at the start, and are done well before the last prefill workgroups.
template <bool F16, bool FP8KV, bool CAUSAL, bool SPLIT, int KG, bool EXT, bool F8MM = false,
          bool MIX = false>
__global__ __launch_bounds__(kWaves * KG * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(const AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[lds_bytes(kWaves * KG)];
    static_assert(!F8MM || (FP8KV && !EXT), "fp8 compute needs an fp8 cache, no mask variants");
    static_assert(!MIX || (!SPLIT && KG == 1), "mixed launches split only the decode rows");
    if constexpr (MIX) {
        const int b = blockIdx.x >> 3, r = blockIdx.x & 7;
        int c0 = a.mix_dblocks;                 // decode blocks placed before block b
        bool dec = false;
        if (b < a.mix_region) {
            c0 = (int)(((int64_t)b * a.mix_dblocks) / a.mix_region);
            dec = (int)(((int64_t)(b + 1) * a.mix_dblocks) / a.mix_region) > c0;
        }
        if (dec) {
            const int d = 8 * c0 + r;           // (sequence x kv head) x split
            if (d >= a.decode_wgs)
                return;
            const int pair = d / a.num_splits;
            decode_body<F16, FP8KV, CAUSAL, true, kWaves, EXT>(a, pair, d - pair * a.num_splits,
                                                               (int)threadIdx.x, lds);
        } else {
            const int pi = 8 * (b - c0) + r;
            if (pi >= a.prefill_wgs)
                return;
            if constexpr (F8MM)
                prefill_body_f8<F16, CAUSAL, false, 1>(a, pi, 0, (int)threadIdx.x, lds);
            else
                prefill_body<F16, FP8KV, CAUSAL, false, 1, EXT>(a, pi, 0, (int)threadIdx.x, lds);
        }
        return;
    }
    if constexpr (SPLIT && KG == 2) {
        // persistent: the workgroups take items i, i + gridDim.x, ... of the
        // (split x (decode, prefill)) grid order, so that items which exit at
        // once do not occupy CUs the working ones are then placed behind
        if (a.persist_items > 0) {
            // odd workgroups take their items in reverse order, so that about
            // half of them start with each kind (streaming decode items
            // then overlap compute-bound prefill items instead of all
            // running at the start or at the end)
            const int n_mine = (a.persist_items - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
            const bool rev = blockIdx.x & 1;
            for (int k = 0;; ++k) {
                // the argument pointer (the kernel-argument segment) and the
                // thread index pass through an empty asm each item, so that the
                // values the bodies derive from them are not hoisted out of the
                // loop to hold registers across it
                using KArgs = const __attribute__((address_space(4))) AttnArgs;
                KArgs *pk = (KArgs *)__builtin_amdgcn_kernarg_segment_ptr();
                asm volatile("" : "+s"(pk));
                const AttnArgs &ai = *(const AttnArgs *)pk;
                int tid = threadIdx.x;
                asm volatile("" : "+v"(tid));
                if (k >= n_mine)
                    break;
                const int it = (int)blockIdx.x + (rev ? n_mine - 1 - k : k) * (int)gridDim.x;
                __syncthreads();                // every wave is done with the last item's LDS
                const int y = it / ai.row_items, x = it - y * ai.row_items;
                if (x < ai.decode_wgs)
                    decode_body<F16, FP8KV, CAUSAL, SPLIT, kWaves * KG, EXT>(ai, x, y, tid, lds);
                else if constexpr (F8MM)
                    prefill_body_f8<F16, CAUSAL, SPLIT, KG>(ai, x - ai.decode_wgs, y, tid, lds);
                else
                    prefill_body<F16, FP8KV, CAUSAL, SPLIT, KG, EXT>(ai, x - ai.decode_wgs, y, tid, lds);
            }
            return;
        }
    }
    const int bx = blockIdx.x;
    if (bx < a.decode_wgs)
        decode_body<F16, FP8KV, CAUSAL, SPLIT, kWaves * KG, EXT>(a, bx, blockIdx.y, (int)threadIdx.x,
                                                                 lds);
    else if constexpr (F8MM)
        prefill_body_f8<F16, CAUSAL, SPLIT, KG>(a, bx - a.decode_wgs, blockIdx.y, (int)threadIdx.x, lds);
    else
        prefill_body<F16, FP8KV, CAUSAL, SPLIT, KG, EXT>(a, bx - a.decode_wgs, blockIdx.y,
                                                         (int)threadIdx.x, lds);
}

// ------------------------------------------------------------------ combine kernel

// One wave per row.  Lane = (split group sg = lane / 16, d chunk c = lane % 16,
// d 8c .. 8c+7): each lane accumulates the splits p = sg, sg + 4, ..., and the
// four split groups are summed with two cross-lane exchanges.  tok_end
// (device, optional): rows of tokens at or past *tok_end belong to no
// sequence; their partials were never written and they are skipped.  The
// running maximum propagates NaN (a split whose key-group barrier timed out
// stores NaN), so such a row's output is NaN rather than a plausible value.
__device__ __forceinline__ float nan_max(float m, float x) { return (x > m || x != x) ? x : m; }

// Merge the P partials of partial row `row` (of `rows` per split) into
// output (tok, head).  One wave per row: every early return is wave-uniform.
template <bool F16>
__device__ __forceinline__ void combine_row(const float *o_part, const float *lse_part, int32_t P,
                                            int64_t rows, int64_t row, int64_t tok, int64_t head,
                                            void *out, int64_t o_st_tok, int64_t o_st_head,
                                            float *lse_out) {
    const int lane = threadIdx.x & 63;
    const int sg = lane >> 4;
    const int c = lane & 15;
    float L = neg_inf();
    for (int p = sg; p < P; p += 4)
        L = nan_max(L, lse_part[(int64_t)p * rows + row]);
    L = nan_max(L, __shfl_xor(L, 16));
    L = nan_max(L, __shfl_xor(L, 32));
    f32x4 a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = a0;
    float wsum = 0.0f;
    if (L != neg_inf()) {
#pragma unroll 2
        for (int p = sg; p < P; p += 4) {
            const int64_t pr = (int64_t)p * rows + row;
            const float w = __builtin_amdgcn_exp2f((lse_part[pr] - L) * kLog2e);
            const f32x4 *src = (const f32x4 *)(o_part + pr * HD + 8 * c);
            a0 += w * src[0];
            a1 += w * src[1];
            wsum += w;
        }
    }
#pragma unroll
    for (int sh = 16; sh <= 32; sh *= 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a0[e] += __shfl_xor(a0[e], sh);
            a1[e] += __shfl_xor(a1[e], sh);
        }
        wsum += __shfl_xor(wsum, sh);
    }
    if (sg != 0)
        return;
    // wsum > 0 is false for NaN as well: a NaN row keeps its NaN sums
    const float inv = wsum > 0.0f ? 1.0f / wsum : (wsum == 0.0f ? 0.0f : wsum);
    uint8_t *op = (uint8_t *)out + (tok * o_st_tok + head * o_st_head + 8 * c) * 2;
    *(u32x4 *)op = u32x4{pack2<F16>(a0[0] * inv, a0[1] * inv), pack2<F16>(a0[2] * inv, a0[3] * inv),
                         pack2<F16>(a1[0] * inv, a1[1] * inv), pack2<F16>(a1[2] * inv, a1[3] * inv)};
    if (lse_out != nullptr && c == 0)
        lse_out[row] = wsum > 0.0f ? L + __logf(wsum) : (wsum == 0.0f ? neg_inf() : wsum);
}

template <bool F16>
__global__ __launch_bounds__(256) void combine_kernel(const float *o_part, const float *lse_part,
                                                      int32_t P, int64_t rows, int32_t Hq, void *out,
                                                      int64_t o_st_tok, int64_t o_st_head,
                                                      float *lse_out, const int32_t *tok_end) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows)
        return;
    const int64_t tok = row / Hq;
    if (tok_end != nullptr && tok >= (int64_t)*tok_end)
        return;
    combine_row<F16>(o_part, lse_part, P, rows, row, tok, row - tok * Hq, out, o_st_tok, o_st_head,
                     lse_out);
}

// The combine of a launch that split only the decode rows: one wave per
// decode row slot (sequence, kv head, row lr < 32 of the decode body's
// (token, head-in-group) numbering); slots of prefill, empty or short
// sequences' missing rows are skipped, their rows written by the prefill
// workgroups or by nobody.
template <bool F16>
__global__ __launch_bounds__(256) void combine_decode_kernel(
    const float *o_part, const float *lse_part, int32_t P, int64_t rows, int32_t Hq, int32_t Hkv,
    int32_t S, const int32_t *cu_seqlens_q, void *out, int64_t o_st_tok, int64_t o_st_head,
    float *lse_out) {
    const int64_t slot = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (slot >= (int64_t)S * Hkv * kDecodeRows)
        return;
    const int lr = (int)(slot % kDecodeRows);
    const int pair = (int)(slot / kDecodeRows);
    const int s = pair / Hkv;
    const int kvh = pair - s * Hkv;
    const int G = Hq / Hkv;
    const int cu0 = cu_seqlens_q[s];
    const int q_len = cu_seqlens_q[s + 1] - cu0;
    if (q_len == 0 || q_len * G > kDecodeRows || lr >= q_len * G)
        return;
    const int tq = lr / G;
    const int64_t tok = (int64_t)cu0 + tq;
    const int64_t head = (int64_t)kvh * G + (lr - tq * G);
    combine_row<F16>(o_part, lse_part, P, rows, tok * Hq + head, tok, head, out, o_st_tok, o_st_head,
                     lse_out);
}

// ------------------------------------------------------------------ launchers

// Launch status: the error state is cleared first, so that an error left by
// an earlier call of the caller's is not reported as this launch's.
template <bool F16, bool FP8KV, bool CAUSAL, bool SPLIT, int KG, bool EXT, bool F8MM = false,
          bool MIX = false>
hipError_t launch_kernel(const AttnArgs &a, dim3 grid, hipStream_t st) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((attn_fwd_kernel<F16, FP8KV, CAUSAL, SPLIT, KG, EXT, F8MM, MIX>), grid,
                       dim3(kWaves * KG * 64), 0, st, a);
    return hipGetLastError();
}

// Two key groups only for split launches; mix: split decode rows only.
template <bool F16, bool FP8KV, bool CAUSAL, bool EXT, bool F8MM = false>
hipError_t launch_shape(const AttnArgs &a, bool split, bool wide, bool mix, dim3 grid, hipStream_t st) {
    if (mix)
        return launch_kernel<F16, FP8KV, CAUSAL, false, 1, EXT, F8MM, true>(a, grid, st);
    if (!split)
        return launch_kernel<F16, FP8KV, CAUSAL, false, 1, EXT, F8MM>(a, grid, st);
    return wide ? launch_kernel<F16, FP8KV, CAUSAL, true, 2, EXT, F8MM>(a, grid, st)
                : launch_kernel<F16, FP8KV, CAUSAL, true, 1, EXT, F8MM>(a, grid, st);
}

template <bool F16, bool FP8KV>
hipError_t launch_mode(const AttnArgs &a, bool causal, bool split, bool wide, bool mix, bool ext,
                       dim3 grid, hipStream_t st) {
    if constexpr (FP8KV) {
        if (a.fp8_compute) {
            if (ext)
                return hipErrorInvalidValue;
            return causal ? launch_shape<F16, true, true, false, true>(a, split, wide, mix, grid, st)
                          : launch_shape<F16, true, false, false, true>(a, split, wide, mix, grid, st);
        }
    }
    if (causal)
        return ext ? launch_shape<F16, FP8KV, true, true>(a, split, wide, mix, grid, st)
                   : launch_shape<F16, FP8KV, true, false>(a, split, wide, mix, grid, st);
    return ext ? launch_shape<F16, FP8KV, false, true>(a, split, wide, mix, grid, st)
               : launch_shape<F16, FP8KV, false, false>(a, split, wide, mix, grid, st);
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, bool q_f16, bool kv_fp8, bool causal, bool split,
                            bool wide, bool mix, dim3 grid, hipStream_t stream) {
    if ((wide && !split) || (mix && (split || a.num_splits < 2 || a.mix_region < a.mix_dblocks ||
                                      grid.y != 1 || (int64_t)grid.x < 8LL * a.mix_dblocks)))
        return hipErrorInvalidValue;
    const bool ext = a.win_left >= 0 || a.win_right >= 0 || a.alibi != nullptr;
    if (q_f16)
        return kv_fp8 ? launch_mode<true, true>(a, causal, split, wide, mix, ext, grid, stream)
                      : launch_mode<true, false>(a, causal, split, wide, mix, ext, grid, stream);
    return kv_fp8 ? launch_mode<false, true>(a, causal, split, wide, mix, ext, grid, stream)
                  : launch_mode<false, false>(a, causal, split, wide, mix, ext, grid, stream);
}

// ------------------------------------------------------------------ no-allocation scratch

// Split partials of ua_unified_attention_noalloc: one array per GPU, held
// until the process ends.  Host code never uses the array's name as an
// address (on the host it is a stand-in, not device memory): the device
// address comes from hipGetSymbolAddress, once per device with that device
// current, and is kept per device.
static __device__ __align__(256) uint8_t scratch[UA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_combine(const float *o_part, const float *lse_part, int32_t num_splits,
                          int64_t rows, int32_t num_q_heads, void *out, bool out_f16,
                          int64_t o_st_tok, int64_t o_st_head, float *lse_out, const int32_t *tok_end,
                          hipStream_t stream) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    (void)hipGetLastError();
    if (out_f16)
        hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, stream, o_part, lse_part,
                           num_splits, rows, num_q_heads, out, o_st_tok, o_st_head, lse_out, tok_end);
    else
        hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, stream, o_part, lse_part,
                           num_splits, rows, num_q_heads, out, o_st_tok, o_st_head, lse_out, tok_end);
    return hipGetLastError();
}

hipError_t launch_combine_decode(const float *o_part, const float *lse_part, int32_t num_splits,
                                 int64_t rows, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t num_seqs, const int32_t *cu_seqlens_q, void *out,
                                 bool out_f16, int64_t o_st_tok, int64_t o_st_head, float *lse_out,
                                 hipStream_t stream) {
    const int64_t slots = (int64_t)num_seqs * num_kv_heads * kDecodeRows;
    const dim3 grid((unsigned)((slots + 3) / 4));
    (void)hipGetLastError();
    if (out_f16)
        hipLaunchKernelGGL(combine_decode_kernel<true>, grid, dim3(256), 0, stream, o_part, lse_part,
                           num_splits, rows, num_q_heads, num_kv_heads, num_seqs, cu_seqlens_q, out,
                           o_st_tok, o_st_head, lse_out);
    else
        hipLaunchKernelGGL(combine_decode_kernel<false>, grid, dim3(256), 0, stream, o_part, lse_part,
                           num_splits, rows, num_q_heads, num_kv_heads, num_seqs, cu_seqlens_q, out,
                           o_st_tok, o_st_head, lse_out);
    return hipGetLastError();
}

}  // namespace ua
