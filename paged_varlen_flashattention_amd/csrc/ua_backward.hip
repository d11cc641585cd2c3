// Attention backward for gfx950 (CDNA4): dQ, dK, dV of packed variable-length
// attention with GQA and the bottom-right causal mask.
//
// What is computed (page "Fused Attention", the tutorial's backward: a
// preprocess forming Delta, a dK/dV loop and a dQ loop, both recomputing P
// from the forward's per-row log-sum-exp), for the loss sum(dO * O):
//   P = exp(scale * Q K^T - LSE),  dV = P^T dO,  dP = dO V^T,
//   Delta_i = sum_d O_id dO_id,  dS = P * (dP - Delta),
//   dQ = scale * dS K,  dK = scale * dS^T Q,
// with a kv head's dK and dV summed over the query heads that read it.
//
// Two kernels, launched in order on one stream:
//   * bwd_dq_kernel: one 4-wave workgroup per (sequence, kv head, block of
//     128 / G query tokens x the G heads), each wave 32 rows with Q and dO in
//     registers, streaming 64-key K and V tiles through LDS as in the forward.
//     It also forms Delta (from the row's O and the dO it holds) and
//     LSE * log2(e) of each of its rows and writes them head-major ([Hq][T])
//     into the workspace, so that 32 consecutive rows of one head are 128
//     contiguous bytes for the second kernel (rows that see no key get +inf,
//     so that their P is exp2(-inf) = 0);
//   * bwd_dkdv_kernel: one 4-wave workgroup per (sequence, kv head, block of
//     128 keys); wave w keeps the K and V rows of its 32 keys in registers as
//     MFMA operands and accumulates dK^T and dV^T (32 keys x 128 d) over every
//     query head of the group and every 32-row query tile that sees its keys.
//     The Q and dO tiles, and their LSE and Delta, go straight from HBM into
//     LDS (global_load_lds), double-buffered, one barrier per tile.
// The two main kernels recompute S and dP each (seven 128-deep products per
// (row, key) pair instead of five); in exchange neither needs atomics.
//
// MFMA 32x32x16 (bf16 / fp16 in, fp32 accumulate) layouts:
//   dK/dV: S = Q K^T and dP = dO V^T with the Q / dO rows fed in a bit-2/3
//   swapped order, so that accumulator register i of lane half h is query row
//   16*(i/8) + 8*h + i%8 of the tile and lane column l%32 is a key: the packed
//   P and dS registers are then directly the B operands of dV^T = dO^T P and
//   dK^T = Q^T dS, whose A operands (dO^T, Q^T) come from transposing LDS
//   reads of the same tiles.
//   dQ: S^T = K Q^T and dP^T = V dO^T (lane column = query row), and
//   dQ^T = K^T dS^T with K^T from transposing reads of the K tile.
// P and dS are rounded to the input dtype for the products (as the tutorial
// does); everything else is fp32.

#include "ua_internal.h"

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

namespace ua {
namespace {

constexpr float kLog2eB = 1.44269504088896341f;
constexpr int kRowBytes = kHeadSize * 2;        // one 16-bit row of 128 values

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// D(32x32) += A(32x16) * B(16x32): lane l holds A row l%32 and B column l%32,
// 8 consecutive k per lane half; D column l%32, rows 8*(r/4) + 4*(l/32) + r%4.
template <bool F16>
__device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <bool F16>
__device__ __forceinline__ uint32_t pk2(float lo, float hi) {
    if constexpr (F16) {
        f16x2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        bf16x2 v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
}

// the two 16-bit values of a word, as fp32 (scalar extraction)
template <bool F16>
__device__ __forceinline__ float lo16(uint32_t w) {
    if constexpr (F16)
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    else
        return __uint_as_float(w << 16);
}
template <bool F16>
__device__ __forceinline__ float hi16(uint32_t w) {
    if constexpr (F16)
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    else
        return __uint_as_float(w & 0xffff0000u);
}

// Swap bits 2 and 3: feeding row sw23(l%32) to MFMA lane row l%32 makes
// accumulator register i of lane half h hold row 16*(i/8) + 8*h + i%8.
__device__ __forceinline__ int sw23(int j) { return (j & ~12) | ((j >> 1) & 4) | ((j << 1) & 8); }

// LDS tiles hold rows of 128 16-bit values (256 bytes, 16 granules of 16 B);
// granule g of row r sits at position g ^ swz(r).  Row reads feed 16 lanes
// the same granule of rows sw23(0..15) (a bijection of r & 15 keeps them on
// 16 distinct positions); transposing reads feed 32 lanes 4 consecutive rows
// x 4 consecutive granules, and swz puts the 4 rows' copies of those granules
// in 4 different groups of 4 positions (its top two bits are r & 3).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ u32x4 row_frag(const uint8_t *t, int row, int gran) {
    return *(const u32x4 *)(t + row * kRowBytes + ((gran ^ swz(row)) << 4));
}

// Transposing 8-byte LDS read: within each 16-lane group, lane i receives
// element i%4 of the 8 bytes addressed by lane 4e + i/4, e = 0..3.
__device__ __forceinline__ u32x2 tr16(const uint8_t *p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                         (__attribute__((address_space(3))) s16x4 *)(p)));
}

// A operand of a product contracting over tile rows 16*kk .. 16*kk+15: lane l
// gets column d = 32*x + l%32 at rows 16*kk + 8*(l/32) + 0..7.
__device__ __forceinline__ u32x4 tr_frag(const uint8_t *t, int kk, int x, int lane) {
    const int jg = lane & 15;
    const int row = 16 * kk + 8 * (lane >> 5) + (jg >> 2);
    const int gran = 4 * x + 2 * ((lane >> 4) & 1) + ((jg & 3) >> 1);
    const u32x2 w0 = tr16(t + row * kRowBytes + ((gran ^ swz(row)) << 4) + 8 * (jg & 1));
    const u32x2 w1 = tr16(t + (row + 4) * kRowBytes + ((gran ^ swz(row + 4)) << 4) + 8 * (jg & 1));
    return u32x4{w0[0], w0[1], w1[0], w1[1]};
}

// 16 (or 4) bytes per lane from global memory straight into LDS: lane l's
// bytes land at lds_row + 16*l (4*l); global address = wave-uniform base +
// per-lane 32-bit offset.  The kernels wait (wait_vm) and synchronise before
// reading what these loads filled.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) {
    return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint8_t *)(p));
}
__device__ __forceinline__ void dma16(const uint8_t *base, uint32_t ofs, uint8_t *lds_row) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(ofs), "s"(base), "s"(lds_addr(lds_row))
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(const uint8_t *base, uint32_t ofs, uint8_t *lds_row) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(ofs), "s"(base), "s"(lds_addr(lds_row))
                 : "memory", "m0");
}
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// s_waitcnt vmcnt(0) as an instruction the compiler's wait bookkeeping
// understands.  That bookkeeping cannot see the inline-asm DMA loads above:
// without this after the prologue, the register operands loaded before the
// tile loop count as in flight at the loop head, and the waits the compiler
// then places for them inside the loop also wait, in hardware, for the next
// tile's DMA issued just before them (the prefetch never overlaps the compute).
__device__ __forceinline__ void vm_settled() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// largest s with cu[s] / B + s <= slot: sequence s owns the slots from
// cu[s] / B + s on (at least ceil(len / B) of them)
__device__ __forceinline__ int find_seq(const int32_t *cu, int num_seqs, int B, int slot) {
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] / B + mid <= slot)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// ------------------------------------------------------------------ dK, dV

constexpr int kRT = 32;                              // query rows per dK/dV tile
constexpr int kKeysPerWg = 128;                      // keys per dK/dV workgroup
constexpr int kDkdvStage = 2 * kRT * kRowBytes + 256;   // Q, dO tiles, 32 LSE2 + 32 Delta

template <bool F16, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(const BwdArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kDkdvStage];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int hl = lane >> 5;
    const int lc = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = a.group;

    const int kvh = blockIdx.x % Hkv;
    const int slot = blockIdx.x / Hkv;
    const int s = find_seq(a.cu_seqlens_k, a.num_seqs, kKeysPerWg, slot);
    const int ck0 = a.cu_seqlens_k[s];
    const int kl = a.cu_seqlens_k[s + 1] - ck0;
    const int kb0 = (slot - (ck0 / kKeysPerWg + s)) * kKeysPerWg;
    if (kb0 >= kl)
        return;                                      // empty slot (uniform)
    const int cq0 = a.cu_seqlens_q[s];
    const int ql = a.cu_seqlens_q[s + 1] - cq0;
    const int ctx = kl - ql;                         // keys before the first query
    const int kw0 = kb0 + 32 * wv;                   // this wave's first key
    const int myk = kw0 + lc;                        // the key of this lane's column
    const bool wave_keys = kw0 < kl;

    // K and V rows of the lane's key: B operands, d = 16*ks + 8*hl + 0..7
    u32x4 kf[8], vf[8];
    {
        const int64_t off = ((int64_t)(ck0 + min(myk, kl - 1)) * Hkv + kvh) * kRowBytes;
        const uint8_t *kp = (const uint8_t *)a.k + off;
        const uint8_t *vp = (const uint8_t *)a.v + off;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            kf[ks] = *(const u32x4 *)(kp + (16 * ks + 8 * hl) * 2);
            vf[ks] = *(const u32x4 *)(vp + (16 * ks + 8 * hl) * 2);
        }
    }

    // row tiles: every query head of the group x the tiles from the first row
    // that sees key kb0 (causal) to the end of the sequence
    const int r_begin = CAUSAL ? (max(0, kb0 - ctx) & ~(kRT - 1)) : 0;
    const int n_rt = ql > r_begin ? (ql - r_begin + kRT - 1) / kRT : 0;
    const int n_it = n_rt * G;
    const float c2 = a.scale * kLog2eB;
    const uint32_t ws_gap = (uint32_t)((const uint8_t *)a.delta - (const uint8_t *)a.lse2);

    auto dma = [&](int it, uint8_t *st) {
        const int hh = it / n_rt;
        const int r0 = r_begin + (it - hh * n_rt) * kRT;
        const int head = kvh * G + hh;
        const int64_t rowb = ((int64_t)(cq0 + r0) * Hq + head) * kRowBytes;
        const uint8_t *qb = (const uint8_t *)a.q + rowb;
        const uint8_t *db = (const uint8_t *)a.dout + rowb;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int rr = 8 * wv + 4 * i + (lane >> 4);             // row within the tile
            const int rc = min(r0 + rr, ql - 1) - r0;                 // rows past the end: a real row
            const uint32_t ofs = (uint32_t)(rc * Hq * kRowBytes) + (uint32_t)(((lane & 15) ^ swz(rr)) << 4);
            dma16(qb, ofs, st + (8 * wv + 4 * i) * kRowBytes);
            dma16(db, ofs, st + kRT * kRowBytes + (8 * wv + 4 * i) * kRowBytes);
        }
        if (wv == 0) {
            // lanes 0..31: LSE2 of rows r0 .. r0+31, lanes 32..63: their Delta
            const uint8_t *lb = (const uint8_t *)(a.lse2 + (int64_t)head * a.num_tokens + cq0);
            const int rc = min(r0 + lc, ql - 1);
            const uint32_t ofs = (uint32_t)rc * 4u + (hl ? ws_gap : 0u);
            dma4(lb, ofs, st + 2 * kRT * kRowBytes);
        }
    };

    f32x16 dkt[4], dvt[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        dkt[x] = f32x16{};
        dvt[x] = f32x16{};
    }
    const int qrow = sw23(lc);

    auto compute = [&](int it, const uint8_t *st) {
        const int hh = it / n_rt;
        const int r0 = r_begin + (it - hh * n_rt) * kRT;
        // uniform: no key of this wave, or no row of the tile sees its first key
        if (!wave_keys || (CAUSAL && ctx + r0 + kRT - 1 < kw0))
            return;
        const uint8_t *sQ = st;
        const uint8_t *sD = st + kRT * kRowBytes;
        const float *sL = (const float *)(st + 2 * kRT * kRowBytes);
        f32x16 sc = f32x16{}, dp = f32x16{};
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            sc = mma<F16>(row_frag(sQ, qrow, 2 * ks + hl), kf[ks], sc);
            dp = mma<F16>(row_frag(sD, qrow, 2 * ks + hl), vf[ks], dp);
        }
        __builtin_amdgcn_s_setprio(0);
        // register i: row r0 + 16*(i/8) + 8*hl + i%8
        float lv[16], dv[16];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const f32x4 l0 = *(const f32x4 *)(sL + 16 * c + 8 * hl);
            const f32x4 l1 = *(const f32x4 *)(sL + 16 * c + 8 * hl + 4);
            const f32x4 d0 = *(const f32x4 *)(sL + 32 + 16 * c + 8 * hl);
            const f32x4 d1 = *(const f32x4 *)(sL + 32 + 16 * c + 8 * hl + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lv[8 * c + e] = l0[e];
                lv[8 * c + 4 + e] = l1[e];
                dv[8 * c + e] = d0[e];
                dv[8 * c + 4 + e] = d1[e];
            }
        }
        const bool masked = r0 + kRT > ql || (CAUSAL && kw0 + 31 > ctx + r0);
        float p[16], ds[16];
        // the tile-level test chooses between two straight copies of the
        // elementwise step (a uniform test inside the loop became a branch
        // per element)
        auto weights = [&](auto masked_c) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float pv = __builtin_amdgcn_exp2f(sc[i] * c2 - lv[i]);
                if constexpr (decltype(masked_c)::value) {
                    const int r = r0 + 16 * (i >> 3) + 8 * hl + (i & 7);
                    if ((r >= ql) | (CAUSAL & (myk > ctx + r)))   // no short-circuit branch
                        pv = 0.0f;
                }
                p[i] = pv;
                ds[i] = pv * (dp[i] - dv[i]);
            }
        };
        if (masked)
            weights(std::true_type{});
        else
            weights(std::false_type{});
        u32x4 pp[2], dd[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            pp[c] = u32x4{pk2<F16>(p[8 * c], p[8 * c + 1]), pk2<F16>(p[8 * c + 2], p[8 * c + 3]),
                          pk2<F16>(p[8 * c + 4], p[8 * c + 5]), pk2<F16>(p[8 * c + 6], p[8 * c + 7])};
            dd[c] = u32x4{pk2<F16>(ds[8 * c], ds[8 * c + 1]), pk2<F16>(ds[8 * c + 2], ds[8 * c + 3]),
                          pk2<F16>(ds[8 * c + 4], ds[8 * c + 5]), pk2<F16>(ds[8 * c + 6], ds[8 * c + 7])};
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                dvt[x] = mma<F16>(tr_frag(sD, c, x, lane), pp[c], dvt[x]);
                dkt[x] = mma<F16>(tr_frag(sQ, c, x, lane), dd[c], dkt[x]);
            }
    };

    uint8_t *const st0 = lds;
    uint8_t *const st1 = lds + kDkdvStage;
    if (n_it > 0) {
        dma(0, st0);
        wait_vm();
        __syncthreads();
    }
    vm_settled();
    auto step = [&](int it, uint8_t *cur, uint8_t *nxt) {
        const bool more = it + 1 < n_it;
        if (more)
            dma(it + 1, nxt);
        compute(it, cur);
        if (more) {
            wait_vm();
            __syncthreads();
        }
    };
    for (int it = 0; it < n_it; it += 2) {
        step(it, st0, st1);
        if (it + 1 < n_it)
            step(it + 1, st1, st0);
    }

    // dK = scale * dK^T, dV = dV^T: lane column = key myk, rows d = 32x + 8g + 4hl + 0..3
    if (myk < kl) {
        const int64_t off = ((int64_t)(ck0 + myk) * Hkv + kvh) * kRowBytes;
        uint8_t *kp = (uint8_t *)a.dk + off;
        uint8_t *vp = (uint8_t *)a.dv + off;
        const float sc = a.scale;
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * x + 8 * g + 4 * hl;
                *(u32x2 *)(kp + d * 2) = u32x2{pk2<F16>(dkt[x][4 * g] * sc, dkt[x][4 * g + 1] * sc),
                                               pk2<F16>(dkt[x][4 * g + 2] * sc, dkt[x][4 * g + 3] * sc)};
                *(u32x2 *)(vp + d * 2) = u32x2{pk2<F16>(dvt[x][4 * g], dvt[x][4 * g + 1]),
                                               pk2<F16>(dvt[x][4 * g + 2], dvt[x][4 * g + 3])};
            }
    }
}

// ------------------------------------------------------------------ dQ

constexpr int kTN = 64;                              // keys per dQ tile
constexpr int kDqStage = 2 * kTN * kRowBytes;        // K and V tiles

template <bool F16, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(const BwdArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kDqStage];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int hl = lane >> 5;
    const int lc = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = a.group;

    const int kvh = blockIdx.x % Hkv;
    int slot = blockIdx.x / Hkv;
    if (CAUSAL)
        slot = a.q_slots - 1 - slot;                 // late (long) query blocks first
    const int s = find_seq(a.cu_seqlens_q, a.num_seqs, a.block_q, slot);
    const int cq0 = a.cu_seqlens_q[s];
    const int ql = a.cu_seqlens_q[s + 1] - cq0;
    const int tq0 = (slot - (cq0 / a.block_q + s)) * a.block_q;
    if (tq0 >= ql)
        return;                                      // empty slot (uniform)
    const int tq1 = min(ql, tq0 + a.block_q);
    const int ck0 = a.cu_seqlens_k[s];
    const int kl = a.cu_seqlens_k[s + 1] - ck0;
    const int ctx = kl - ql;

    // rows: wave w holds rows 32w .. 32w+31 of the block, row r = token r / G, head r % G
    const int r = 32 * wv + lc;
    const int tq = r / G;
    const int head = kvh * G + (r - tq * G);
    const bool row_ok = tq0 + tq < tq1;
    const int64_t tok = (int64_t)cq0 + tq0 + tq;
    const int lim = !row_ok ? 0 : (CAUSAL ? min(kl, ctx + tq0 + tq + 1) : kl);
    u32x4 qf[8], df[8];
    float lse2 = __builtin_inff(), delta = 0.0f;
    if (row_ok) {
        const int64_t off = (tok * Hq + head) * kRowBytes;
        const uint8_t *qp = (const uint8_t *)a.q + off;
        const uint8_t *dp = (const uint8_t *)a.dout + off;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            qf[ks] = *(const u32x4 *)(qp + (16 * ks + 8 * hl) * 2);
            df[ks] = *(const u32x4 *)(dp + (16 * ks + 8 * hl) * 2);
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            qf[ks] = u32x4{0, 0, 0, 0};
            df[ks] = u32x4{0, 0, 0, 0};
        }
    }
    // Delta = sum_d O dO of the row: each lane half holds the dO values of
    // half the row's d (8 per k-step), the matching O values are read here;
    // LSE * log2(e) from the forward's natural-log LSE.  Both go to the
    // workspace for the dK/dV kernel (one lane per row).
    {
        float part = 0.0f;
        if (row_ok) {
            const uint8_t *op = (const uint8_t *)a.o + (tok * Hq + head) * kRowBytes;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const u32x4 o = *(const u32x4 *)(op + (16 * ks + 8 * hl) * 2);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    part += lo16<F16>(o[e]) * lo16<F16>(df[ks][e]) + hi16<F16>(o[e]) * hi16<F16>(df[ks][e]);
            }
        }
        const float dsum = part + __shfl_xor(part, 32);     // the other lane half of the row
        if (row_ok) {
            const float l = a.lse[tok * Hq + head];
            lse2 = l == -__builtin_inff() ? __builtin_inff() : l * kLog2eB;
            delta = dsum;
            if (hl == 0) {
                a.lse2[(int64_t)head * a.num_tokens + tok] = lse2;
                a.delta[(int64_t)head * a.num_tokens + tok] = delta;
            }
        }
    }

    // keys seen by some row / by every row of the block
    const int kv_end = CAUSAL ? min(kl, ctx + tq1) : kl;
    const int full_end = CAUSAL ? min(kl, ctx + tq0 + 1) : kl;
    const int n_tiles = max(kv_end, 0) / kTN + ((max(kv_end, 0) % kTN) != 0);
    const int n_full = max(full_end, 0) / kTN;
    const float c2 = a.scale * kLog2eB;

    const uint8_t *kbase = (const uint8_t *)a.k + ((int64_t)ck0 * Hkv + kvh) * kRowBytes;
    const uint8_t *vbase = (const uint8_t *)a.v + ((int64_t)ck0 * Hkv + kvh) * kRowBytes;
    auto dma = [&](int t, uint8_t *st) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = 16 * wv + 4 * i + (lane >> 4);            // key row within the tile
            const int key = min(t * kTN + rr, kl - 1);               // keys past the end: a real key
            const uint32_t ofs = (uint32_t)(key * Hkv * kRowBytes) + (uint32_t)(((lane & 15) ^ swz(rr)) << 4);
            dma16(kbase, ofs, st + (16 * wv + 4 * i) * kRowBytes);
            dma16(vbase, ofs, st + kTN * kRowBytes + (16 * wv + 4 * i) * kRowBytes);
        }
    };

    f32x16 dqt[4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
        dqt[x] = f32x16{};
    const bool wave_on = 32 * wv < (tq1 - tq0) * G;  // uniform

    auto compute = [&](int t, const uint8_t *st) {
        if (!wave_on)
            return;
        const uint8_t *sK = st;
        const uint8_t *sV = st + kTN * kRowBytes;
        f32x16 sc[2], dp[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            sc[b] = f32x16{};
            dp[b] = f32x16{};
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int kr = 32 * b + sw23(lc);
                sc[b] = mma<F16>(row_frag(sK, kr, 2 * ks + hl), qf[ks], sc[b]);
                dp[b] = mma<F16>(row_frag(sV, kr, 2 * ks + hl), df[ks], dp[b]);
            }
        __builtin_amdgcn_s_setprio(0);
        // register i of block b: key t*64 + 32b + 16*(i/8) + 8*hl + i%8
        const bool masked = t >= n_full;
        u32x4 dd[4];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            float ds[16];
            // two straight copies of the elementwise step, chosen per tile
            auto weights = [&](auto masked_c) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float pv = __builtin_amdgcn_exp2f(sc[b][i] * c2 - lse2);
                    if constexpr (decltype(masked_c)::value) {
                        const int j = t * kTN + 32 * b + 16 * (i >> 3) + 8 * hl + (i & 7);
                        if (j >= lim)
                            pv = 0.0f;
                    }
                    ds[i] = pv * (dp[b][i] - delta);
                }
            };
            if (masked)
                weights(std::true_type{});
            else
                weights(std::false_type{});
#pragma unroll
            for (int c = 0; c < 2; ++c)
                dd[2 * b + c] = u32x4{pk2<F16>(ds[8 * c], ds[8 * c + 1]), pk2<F16>(ds[8 * c + 2], ds[8 * c + 3]),
                                      pk2<F16>(ds[8 * c + 4], ds[8 * c + 5]), pk2<F16>(ds[8 * c + 6], ds[8 * c + 7])};
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int x = 0; x < 4; ++x)
                dqt[x] = mma<F16>(tr_frag(sK, kk, x, lane), dd[kk], dqt[x]);
    };

    uint8_t *const st0 = lds;
    uint8_t *const st1 = lds + kDqStage;
    if (n_tiles > 0) {
        dma(0, st0);
        wait_vm();
        __syncthreads();
    }
    vm_settled();
    auto step = [&](int t, uint8_t *cur, uint8_t *nxt) {
        const bool more = t + 1 < n_tiles;
        if (more)
            dma(t + 1, nxt);
        compute(t, cur);
        if (more) {
            wait_vm();
            __syncthreads();
        }
    };
    for (int t = 0; t < n_tiles; t += 2) {
        step(t, st0, st1);
        if (t + 1 < n_tiles)
            step(t + 1, st1, st0);
    }

    // dQ = scale * dQ^T: lane column = row (tok, head), rows d = 32x + 8g + 4hl + 0..3
    if (row_ok) {
        uint8_t *qp = (uint8_t *)a.dq + (tok * Hq + head) * kRowBytes;
        const float sc = a.scale;
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * x + 8 * g + 4 * hl;
                *(u32x2 *)(qp + d * 2) = u32x2{pk2<F16>(dqt[x][4 * g] * sc, dqt[x][4 * g + 1] * sc),
                                               pk2<F16>(dqt[x][4 * g + 2] * sc, dqt[x][4 * g + 3] * sc)};
            }
    }
}

template <bool F16, bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t st) {
    hipError_t e = hipSuccess;
    (void)hipGetLastError();                    // report these launches' status only
    // dQ first: it writes the Delta and LSE * log2(e) rows dK/dV reads
    if (a.dq_wgs > 0) {
        hipLaunchKernelGGL((bwd_dq_kernel<F16, CAUSAL>), dim3((unsigned)a.dq_wgs), dim3(256), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    if (a.dkdv_wgs > 0) {
        hipLaunchKernelGGL((bwd_dkdv_kernel<F16, CAUSAL>), dim3((unsigned)a.dkdv_wgs), dim3(256), 0, st, a);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

hipError_t launch_backward(const BwdArgs &a, bool f16, bool causal, hipStream_t stream) {
    if (f16)
        return causal ? launch_bwd_t<true, true>(a, stream) : launch_bwd_t<true, false>(a, stream);
    return causal ? launch_bwd_t<false, true>(a, stream) : launch_bwd_t<false, false>(a, stream);
}

}  // namespace ua
