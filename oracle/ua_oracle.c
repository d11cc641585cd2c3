/*
 * ua_oracle.c -- plain CPU fp64 oracle for paged, variable-length attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU library: its own decoding, its own
 * indexing and its own loops.
 *
 * What it computes is the plain definition of attention over a KV cache
 * (page "flashatten takeaways EP2 工程", section "kv cache", the boxed formula
 * O = softmax(q K^T / sqrt(d)) V over all cached tokens), with
 *   - packed queries addressed through cu_seqlens_q (page "vLLM Triton unified
 *     attention notes", section test_triton_unified_attn: an inclusive prefix
 *     sum of the query lengths, read here with a leading 0);
 *   - the KV cache [num_blocks, block_size, kv_heads, head_size] read through
 *     one page table per sequence (same page, sections test_triton_unified_attn
 *     and kernel_unified_attention_2d: physical block = block_table[s][pos /
 *     block_size], slot = pos % block_size, four element strides);
 *   - GQA: query head h reads kv head h / (Hq / Hkv) (same page, section
 *     kernel_unified_attention_2d, the proof that the largest query head index
 *     is Hq - 1);
 *   - causal masking with the queries at the end of the sequence: query i of a
 *     sequence with q_len queries and kv_len keys sits at absolute position
 *     kv_len - q_len + i and sees keys 0 .. kv_len - q_len + i (same section:
 *     context_len is the number of tokens before the current queries);
 *   - fp8 KV values dequantised as code * scale (same section: K and V are
 *     loaded, then dequantised with their per-tensor scales);
 *   - optional local (sliding-window) attention and ALiBi bias, the two
 *     switches of the FA2 forward launch (page "flashatten takeaways EP2 工程",
 *     section "源代码接口": window_size_left / window_size_right and
 *     alibi_slopes_ptr).  The pages name the switches but not their formulas;
 *     the reading taken here is the usual one: with the query at absolute
 *     position pos, keys pos - window_left .. pos + window_right are visible (a
 *     negative bound is no bound), and the logit of key j gets
 *     -slope[h] * |pos - j| added after the softmax scale.
 * It is computed in double precision, with exp/log from libm, summed in
 * key order.  No blocking, no online rescaling, no split.
 *
 * The split combine (uao_combine) is the log-sum-exp merge of partial results
 * (page "flashatten takeaways EP2 工程", section "源代码接口": the split-KV
 * interface first stores per-split partial results, then a combine kernel
 * corrects them into the exact result; page "Fused Attention", section
 * FlashDecoding: split K/V into chunks, attend to each, then a global reduce).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { UAO_BF16 = 0, UAO_FP16 = 1, UAO_FP8_E4M3FN = 2, UAO_F64 = 3 };

/* ---------------------------------------------------------------- decoding */

/* bfloat16: the top 16 bits of an IEEE-754 binary32. */
static double dec_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE-754 binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
static double dec_fp16(uint16_t bits)
{
    int sign = bits >> 15;
    int e = (bits >> 10) & 0x1f;
    int m = bits & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);               /* m/2^10 * 2^(1-15) */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);   /* (1 + m/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* OCP 8-bit floating point, E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa
 * bits; no infinities; S.1111.111 is NaN; largest finite magnitude 448. */
static double dec_e4m3fn(uint8_t bits)
{
    int sign = bits >> 7;
    int e = (bits >> 3) & 0xf;
    int m = bits & 0x7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);                /* m/8 * 2^(1-7) */
    else
        v = ldexp((double)(8 + m), e - 10);      /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

static double load(const void *base, int dtype, int64_t idx)
{
    switch (dtype) {
    case UAO_BF16: return dec_bf16(((const uint16_t *)base)[idx]);
    case UAO_FP16: return dec_fp16(((const uint16_t *)base)[idx]);
    case UAO_FP8_E4M3FN: return dec_e4m3fn(((const uint8_t *)base)[idx]);
    case UAO_F64: return ((const double *)base)[idx];   /* queries given as exact doubles */
    default: return NAN;
    }
}

/* Decode n stored values of the given dtype to double (used to pin the tables). */
int uao_decode(int dtype, const void *src, double *dst, int64_t n)
{
    if (dtype < UAO_BF16 || dtype > UAO_FP8_E4M3FN)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        dst[i] = load(src, dtype, i);
    return 0;
}

/* ---------------------------------------------------------------- attention */

typedef struct {
    const void *q; int q_dtype; int64_t q_st_tok, q_st_head;
    const void *k; const void *v; int kv_dtype;
    int64_t kv_st_blk, kv_st_slot, kv_st_head;
    const int32_t *cu_seqlens_q, *seqused_k, *block_table; int64_t bt_stride;
    int32_t num_seqs, num_q_heads, num_kv_heads, head_size, block_size;
    double scale; int causal; double k_scale, v_scale;
    int32_t kv_lo, kv_hi;
    int32_t win_left, win_right;                  /* < 0: no bound on that side */
    const double *alibi;                          /* [num_q_heads] slopes, or NULL */
} problem;

/* Element offset of (logical key position pos, kv head g, dim d) of sequence s. */
static int64_t kv_offset(const problem *p, int32_t s, int32_t pos, int32_t g, int32_t d)
{
    int32_t blk = p->block_table[(int64_t)s * p->bt_stride + pos / p->block_size];
    int32_t slot = pos % p->block_size;
    return (int64_t)blk * p->kv_st_blk + (int64_t)slot * p->kv_st_slot
         + (int64_t)g * p->kv_st_head + d;
}

/* One output row: token t (packed index), query head h. */
static void one_row(const problem *p, int64_t t, int32_t h, double *out, double *lse)
{
    const int32_t D = p->head_size;
    int32_t s = 0;
    while (s < p->num_seqs && !(p->cu_seqlens_q[s] <= t && t < p->cu_seqlens_q[s + 1]))
        ++s;
    for (int32_t d = 0; d < D; ++d)
        out[d] = 0.0;
    *lse = -INFINITY;
    if (s == p->num_seqs)
        return;                                   /* token outside every sequence */

    const int32_t q_len = p->cu_seqlens_q[s + 1] - p->cu_seqlens_q[s];
    const int32_t kv_len = p->seqused_k[s];
    const int32_t i = (int32_t)(t - p->cu_seqlens_q[s]);
    const int32_t ctx = kv_len - q_len;           /* keys before the first query */
    const int32_t g = h / (p->num_q_heads / p->num_kv_heads);

    /* visible keys: [0, kv_len), and j <= ctx + i when causal, intersected with
       [kv_lo, kv_hi) when a partial result over a key range is asked for */
    const int32_t pos = ctx + i;                  /* absolute position of the query */
    int32_t lo = 0, hi = kv_len;
    if (p->causal && ctx + i + 1 < hi)
        hi = ctx + i + 1;
    if (p->win_left >= 0 && pos - p->win_left > lo)
        lo = pos - p->win_left;
    if (p->win_right >= 0 && pos + p->win_right + 1 < hi)
        hi = pos + p->win_right + 1;
    if (p->kv_lo > lo)
        lo = p->kv_lo;
    if (p->kv_hi >= 0 && p->kv_hi < hi)
        hi = p->kv_hi;
    if (hi <= lo)
        return;                                   /* no visible key: o = 0, lse = -inf */

    double *qv = malloc(sizeof(double) * D);
    double *z = malloc(sizeof(double) * (size_t)(hi - lo));
    for (int32_t d = 0; d < D; ++d)
        qv[d] = load(p->q, p->q_dtype, t * p->q_st_tok + (int64_t)h * p->q_st_head + d);

    /* scores z_j = scale * q . k_j */
    double m = -INFINITY;
    for (int32_t j = lo; j < hi; ++j) {
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d)
            dot += qv[d] * (load(p->k, p->kv_dtype, kv_offset(p, s, j, g, d)) * p->k_scale);
        z[j - lo] = p->scale * dot;
        if (p->alibi)
            z[j - lo] -= p->alibi[h] * fabs((double)(pos - j));
        if (z[j - lo] > m)
            m = z[j - lo];
    }
    /* softmax-weighted sum of the value rows */
    double denom = 0.0;
    for (int32_t j = lo; j < hi; ++j) {
        double w = exp(z[j - lo] - m);
        denom += w;
        for (int32_t d = 0; d < D; ++d)
            out[d] += w * (load(p->v, p->kv_dtype, kv_offset(p, s, j, g, d)) * p->v_scale);
    }
    for (int32_t d = 0; d < D; ++d)
        out[d] /= denom;
    *lse = m + log(denom);
    free(z);
    free(qv);
}

/*
 * Attention rows.  rows holds n_rows (token, head) pairs as int64; when rows is
 * NULL every (token, head) of the batch is computed in token-major order and
 * n_rows must equal num_tokens * num_q_heads.  out is [n_rows, head_size],
 * lse is [n_rows] (natural log of the softmax denominator, max included).
 * kv_lo / kv_hi (kv_hi < 0: no upper bound) restrict the keys to a range of
 * absolute positions, which yields the partial result of one split.
 * win_left / win_right (< 0: unbounded) give local attention, alibi_slopes
 * ([num_q_heads] or NULL) the ALiBi bias (see the header).
 * Returns 0, or -1 on an invalid argument.
 */
int uao_attention_ex(const void *q, int q_dtype, int64_t q_st_tok, int64_t q_st_head,
                     const void *k_cache, const void *v_cache, int kv_dtype,
                     int64_t kv_st_blk, int64_t kv_st_slot, int64_t kv_st_head,
                     const int32_t *cu_seqlens_q, const int32_t *seqused_k,
                     const int32_t *block_table, int64_t bt_stride,
                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_size, int32_t block_size,
                     double softmax_scale, int causal, double k_scale, double v_scale,
                     int32_t kv_lo, int32_t kv_hi,
                     int32_t win_left, int32_t win_right, const double *alibi_slopes,
                     const int64_t *rows, int64_t n_rows,
                     double *out, double *lse, int nthreads)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0)
        return -1;
    if (num_q_heads % num_kv_heads != 0)
        return -1;
    problem p = {q, q_dtype, q_st_tok, q_st_head, k_cache, v_cache, kv_dtype,
                 kv_st_blk, kv_st_slot, kv_st_head, cu_seqlens_q, seqused_k, block_table, bt_stride,
                 num_seqs, num_q_heads, num_kv_heads, head_size, block_size,
                 softmax_scale, causal, k_scale, v_scale, kv_lo, kv_hi,
                 win_left, win_right, alibi_slopes};
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t t = rows ? rows[2 * r] : r / num_q_heads;
        int32_t h = (int32_t)(rows ? rows[2 * r + 1] : r % num_q_heads);
        one_row(&p, t, h, out + r * head_size, lse + r);
    }
    return 0;
}

/* uao_attention_ex without local attention or ALiBi. */
int uao_attention(const void *q, int q_dtype, int64_t q_st_tok, int64_t q_st_head,
                  const void *k_cache, const void *v_cache, int kv_dtype,
                  int64_t kv_st_blk, int64_t kv_st_slot, int64_t kv_st_head,
                  const int32_t *cu_seqlens_q, const int32_t *seqused_k,
                  const int32_t *block_table, int64_t bt_stride,
                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                  int32_t head_size, int32_t block_size,
                  double softmax_scale, int causal, double k_scale, double v_scale,
                  int32_t kv_lo, int32_t kv_hi,
                  const int64_t *rows, int64_t n_rows,
                  double *out, double *lse, int nthreads)
{
    return uao_attention_ex(q, q_dtype, q_st_tok, q_st_head, k_cache, v_cache, kv_dtype,
                            kv_st_blk, kv_st_slot, kv_st_head, cu_seqlens_q, seqused_k,
                            block_table, bt_stride, num_seqs, num_q_heads, num_kv_heads,
                            head_size, block_size, softmax_scale, causal, k_scale, v_scale,
                            kv_lo, kv_hi, -1, -1, NULL, rows, n_rows, out, lse, nthreads);
}

/*
 * Combine per-split partial results: for each row, partial p holds the
 * normalised output o_p[head_size] and its log-sum-exp lse_p (natural log).
 * out = sum_p exp(lse_p - L) o_p / sum_p exp(lse_p - L) with L = max_p lse_p,
 * lse = L + log(sum_p exp(lse_p - L)).  Splits with lse_p = -inf weigh 0; a row
 * whose splits are all empty gives out = 0, lse = -inf.
 * o_part is [num_splits, n_rows, head_size], lse_part is [num_splits, n_rows].
 */
int uao_combine(const double *o_part, const double *lse_part, int32_t num_splits,
                int64_t n_rows, int32_t head_size, double *out, double *lse)
{
    if (num_splits < 1 || n_rows < 0 || head_size <= 0)
        return -1;
    for (int64_t r = 0; r < n_rows; ++r) {
        double L = -INFINITY;
        for (int32_t sp = 0; sp < num_splits; ++sp)
            if (lse_part[(int64_t)sp * n_rows + r] > L)
                L = lse_part[(int64_t)sp * n_rows + r];
        for (int32_t d = 0; d < head_size; ++d)
            out[r * head_size + d] = 0.0;
        if (L == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double wsum = 0.0;
        for (int32_t sp = 0; sp < num_splits; ++sp) {
            double w = exp(lse_part[(int64_t)sp * n_rows + r] - L);
            wsum += w;
            for (int32_t d = 0; d < head_size; ++d)
                out[r * head_size + d] += w * o_part[((int64_t)sp * n_rows + r) * head_size + d];
        }
        for (int32_t d = 0; d < head_size; ++d)
            out[r * head_size + d] /= wsum;
        lse[r] = L + log(wsum);
    }
    return 0;
}
