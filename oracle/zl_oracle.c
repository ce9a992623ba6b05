/*
 * zl_oracle.c -- plain fp64 CPU oracle for fused batched decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this file's library.  The GPU library
 * shares no code, header, table or helper with it, and never calls it.
 *
 * What is computed (the pages print no formula; this is the plain reading):
 *   ZhiLight's decode stage attends one new query token per head, for every
 *   sequence of a dynamically assembled batch, over that sequence's cache
 *   ("ZhiLight: 知乎开源的高性能 LLM 推理加速引擎", section 4 "Tensor Core 上的
 *   Flash Attention"; "ZhiLight: Zhihu's CUDA Inference Engine ...", section
 *   "Dual streams, host all-reduce and the memory model").  The batch holds
 *   requests of different lengths (first page, section "功能生态", dynamic
 *   batching).  Query heads may share a key/value head (third page, part 01
 *   section 1, Multi-Query Attention).  Fused, flash or split-KV attention all
 *   reach the plain scaled-dot-product result up to rounding, so the oracle is
 *   that definition written out:
 *
 *     s_i   = scale * sum_d q[d] * K[i][d]          (i < L, fp64, in order)
 *     m     = max_i s_i
 *     w_i   = exp(s_i - m),   l = sum_i w_i
 *     out[e]= (sum_i w_i * V[i][e]) / l
 *     lse   = m + ln(l)                              (natural log)
 *     L = 0: out = 0, lse = -inf
 *
 *   Every 16-bit input element is decoded exactly to double before use.
 *
 * MLA (DeepSeek-V2 multi-head latent attention, named on the first page,
 * sections "技术架构" and "功能生态", and on the second page's "Dual streams"
 * section) is read as the absorbed form: one latent row of 576 values per
 * token (512 latent + 64 rotary), every query head attends over the whole row
 * with a query already multiplied into latent space, and the value is the
 * first 512 columns of the same row.  It is the routine above with one
 * key/value head, K = row[0:576], V = row[0:512].
 *
 * The log-sum-exp combine merges per-split partial results (normalised
 * output O_s and lse_s of disjoint token subsets) into the result over their
 * union:  M = max_s lse_s,  w_s = exp(lse_s - M),
 *         out = sum_s w_s O_s / sum_s w_s,  lse = M + ln(sum_s w_s);
 *         all lse_s = -inf  ->  out = 0, lse = -inf.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ZO_F16 0
#define ZO_BF16 1

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
double zo_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);             /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25); /* (1.m) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double zo_bf16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int m = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);            /* subnormal: m * 2^(-126-7) */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x80), e - 134); /* (1.m) * 2^(e-127) */
    return sign ? -v : v;
}

/* The two decoders above, memoised for all 65,536 patterns when the library
 * loads (a lookup returns exactly the value the function computes). */
static double f16_values[65536];
static double bf16_values[65536];

__attribute__((constructor)) static void zo_fill_decode_tables(void)
{
    for (int i = 0; i < 65536; ++i) {
        f16_values[i] = zo_f16_to_f64((uint16_t)i);
        bf16_values[i] = zo_bf16_to_f64((uint16_t)i);
    }
}

static double dec(uint16_t h, int dtype)
{
    return dtype == ZO_BF16 ? bf16_values[h] : f16_values[h];
}

/* One query row against L key/value rows.  s is scratch of at least L + dk
 * doubles (the weights, then the decoded query row). */
static void attend_one(const uint16_t *q, const uint16_t *k, long k_stride,
                       const uint16_t *v, long v_stride, int L, int dk, int dv,
                       double scale, int dtype, double *out, double *lse,
                       double *s)
{
    if (L <= 0) {
        for (int e = 0; e < dv; ++e)
            out[e] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double *qd = s + L;
    for (int d = 0; d < dk; ++d)
        qd[d] = dec(q[d], dtype);
    for (int i = 0; i < L; ++i) {
        double acc = 0.0;
        for (int d = 0; d < dk; ++d)
            acc += qd[d] * dec(k[(long)i * k_stride + d], dtype);
        s[i] = scale * acc;
    }
    double m = s[0];
    for (int i = 1; i < L; ++i)
        if (s[i] > m)
            m = s[i];
    double l = 0.0;
    for (int i = 0; i < L; ++i) {
        s[i] = exp(s[i] - m); /* s now holds the weights w_i */
        l += s[i];
    }
    /* out[e] = (sum over i, in order, of w_i * V[i][e]) / l; the rows of V
     * are walked in token order, each adding its term to every out[e]. */
    for (int e = 0; e < dv; ++e)
        out[e] = 0.0;
    for (int i = 0; i < L; ++i) {
        const uint16_t *vrow = v + (long)i * v_stride;
        for (int e = 0; e < dv; ++e)
            out[e] += s[i] * dec(vrow[e], dtype);
    }
    for (int e = 0; e < dv; ++e)
        out[e] /= l;
    *lse = m + log(l);
}

/*
 * General decode attention over a packed ragged cache.
 *   q   : [batch, num_q_heads, dk]
 *   K(t, g, d) = k[t * k_row_stride + g * dk + d]
 *   V(t, g, e) = v[t * v_row_stride + g * dv + e]
 *   cu  : [batch + 1], sequence b owns rows cu[b] .. cu[b+1]-1
 *   query head h reads key/value head h / (num_q_heads / num_kv_heads)
 *   pairs: optional list of npairs (b, h) to compute; NULL = all pairs.
 *   out : [batch, num_q_heads, dv],  lse : [batch, num_q_heads]
 * Returns 0, or -1 on a bad argument.
 */
int zo_decode_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   const int32_t *cu, int batch, int num_q_heads,
                   int num_kv_heads, int dk, int dv, long k_row_stride,
                   long v_row_stride, double scale, int dtype,
                   const int32_t *pairs, int npairs, double *out, double *lse,
                   int nthreads)
{
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || dk <= 0 ||
        dv <= 0 || num_q_heads % num_kv_heads != 0)
        return -1;
    int group = num_q_heads / num_kv_heads;
    long total = pairs ? (long)npairs : (long)batch * num_q_heads;
    int max_len = 0;
    for (int b = 0; b < batch; ++b) {
        int L = cu[b + 1] - cu[b];
        if (L < 0)
            return -1;
        if (L > max_len)
            max_len = L;
    }
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * ((size_t)max_len + (size_t)dk));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long p = 0; p < total; ++p) {
            if (!s)
                continue;
            int b = pairs ? pairs[2 * p] : (int)(p / num_q_heads);
            int h = pairs ? pairs[2 * p + 1] : (int)(p % num_q_heads);
            if (b < 0 || b >= batch || h < 0 || h >= num_q_heads)
                continue;
            int g = h / group;
            int L = cu[b + 1] - cu[b];
            attend_one(q + ((long)b * num_q_heads + h) * dk,
                       k + (long)cu[b] * k_row_stride + (long)g * dk, k_row_stride,
                       v + (long)cu[b] * v_row_stride + (long)g * dv, v_row_stride,
                       L, dk, dv, scale, dtype,
                       out + ((long)b * num_q_heads + h) * dv,
                       lse + (long)b * num_q_heads + h, s);
        }
        free(s);
    }
    return bad ? -1 : 0;
}

/*
 * Attention of several new query tokens per sequence (chunked prefill, or
 * several draft tokens verified at once).  The first ZhiLight page lists
 * chunked prefill among the engine's features (section "功能生态"), and the
 * second page lists it beside flash-attention prefill (section "Dual streams,
 * host all-reduce and the memory model").  Sequence b has Lq = cu_q[b+1] -
 * cu_q[b] new query tokens, whose keys and values are already the last Lq of
 * its Lk = cu_k[b+1] - cu_k[b] cached rows.  New token i (0 <= i < Lq) sits at
 * cache position Lk - Lq + i; with `causal` it attends to cache rows
 * 0 .. Lk - Lq + i (none when that is negative), otherwise to all Lk rows.
 * Each query row is then the decode definition above over its visible rows.
 *   q   : [total_q, num_q_heads, dk],  K/V as in zo_decode_attn with cu_k
 *   rows: optional list of nrows (t, h) query rows to compute; NULL = all.
 *   out : [total_q, num_q_heads, dv],  lse : [total_q, num_q_heads]
 */
int zo_varlen_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   const int32_t *cu_q, const int32_t *cu_k, int batch,
                   int num_q_heads, int num_kv_heads, int dk, int dv,
                   long k_row_stride, long v_row_stride, double scale,
                   int causal, int dtype, const int32_t *rows, int nrows,
                   double *out, double *lse, int nthreads)
{
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || dk <= 0 ||
        dv <= 0 || num_q_heads % num_kv_heads != 0 || cu_q[0] != 0)
        return -1;
    int group = num_q_heads / num_kv_heads;
    int max_len = 0;
    for (int b = 0; b < batch; ++b) {
        int Lq = cu_q[b + 1] - cu_q[b], Lk = cu_k[b + 1] - cu_k[b];
        if (Lq < 0 || Lk < 0)
            return -1;
        if (Lk > max_len)
            max_len = Lk;
    }
    long total_q = cu_q[batch];
    long total = rows ? (long)nrows : total_q * num_q_heads;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * ((size_t)max_len + (size_t)dk));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long p = 0; p < total; ++p) {
            if (!s)
                continue;
            long t = rows ? rows[2 * p] : p / num_q_heads;
            int h = rows ? rows[2 * p + 1] : (int)(p % num_q_heads);
            if (t < 0 || t >= total_q || h < 0 || h >= num_q_heads)
                continue;
            int b = 0; /* the sequence holding query token t */
            while (cu_q[b + 1] <= t)
                ++b;
            int Lq = cu_q[b + 1] - cu_q[b], Lk = cu_k[b + 1] - cu_k[b];
            int i = (int)(t - cu_q[b]);
            int L = causal ? Lk - Lq + i + 1 : Lk;
            if (L < 0)
                L = 0;
            if (L > Lk)
                L = Lk;
            int g = h / group;
            attend_one(q + (t * num_q_heads + h) * dk,
                       k + (long)cu_k[b] * k_row_stride + (long)g * dk, k_row_stride,
                       v + (long)cu_k[b] * v_row_stride + (long)g * dv, v_row_stride,
                       L, dk, dv, scale, dtype,
                       out + (t * num_q_heads + h) * dv,
                       lse + t * num_q_heads + h, s);
        }
        free(s);
    }
    return bad ? -1 : 0;
}

/* GQA/MQA/MHA: K and V are [total_tokens, num_kv_heads, head_dim]. */
int zo_gqa_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  const int32_t *cu, int batch, int num_q_heads,
                  int num_kv_heads, int head_dim, double scale, int dtype,
                  const int32_t *pairs, int npairs, double *out, double *lse,
                  int nthreads)
{
    long stride = (long)num_kv_heads * head_dim;
    return zo_decode_attn(q, k, v, cu, batch, num_q_heads, num_kv_heads,
                          head_dim, head_dim, stride, stride, scale, dtype,
                          pairs, npairs, out, lse, nthreads);
}

/* Absorbed MLA: latent rows [total_tokens, kv_lora_rank + rope_dim];
 * K = whole row, V = first kv_lora_rank columns of the same row. */
int zo_mla_decode(const uint16_t *q, const uint16_t *latent, const int32_t *cu,
                  int batch, int num_q_heads, int kv_lora_rank, int rope_dim,
                  double scale, int dtype, const int32_t *pairs, int npairs,
                  double *out, double *lse, int nthreads)
{
    int row = kv_lora_rank + rope_dim;
    return zo_decode_attn(q, latent, latent, cu, batch, num_q_heads, 1, row,
                          kv_lora_rank, row, row, scale, dtype, pairs, npairs,
                          out, lse, nthreads);
}

/* Log-sum-exp combine of num_splits partial results.
 *   part_out : [num_splits, rows, dv] (normalised),  part_lse : [num_splits, rows]
 *   out : [rows, dv],  lse : [rows]                                    */
void zo_combine(const double *part_out, const double *part_lse, int num_splits,
                long rows, int dv, double *out, double *lse)
{
    for (long r = 0; r < rows; ++r) {
        double M = -INFINITY;
        for (int s = 0; s < num_splits; ++s)
            if (part_lse[(long)s * rows + r] > M)
                M = part_lse[(long)s * rows + r];
        if (M == -INFINITY) {
            for (int e = 0; e < dv; ++e)
                out[r * dv + e] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        double wsum = 0.0;
        for (int s = 0; s < num_splits; ++s)
            wsum += exp(part_lse[(long)s * rows + r] - M);
        for (int e = 0; e < dv; ++e) {
            double acc = 0.0;
            for (int s = 0; s < num_splits; ++s) {
                if (part_lse[(long)s * rows + r] == -INFINITY)
                    continue; /* an empty split carries no weight */
                double w = exp(part_lse[(long)s * rows + r] - M);
                acc += w * part_out[((long)s * rows + r) * dv + e];
            }
            out[r * dv + e] = acc / wsum;
        }
        lse[r] = M + log(wsum);
    }
}

int zo_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Decode n 16-bit values to double (used to pin the decoders). */
void zo_decode_array(const uint16_t *in, long n, int dtype, double *out)
{
    for (long i = 0; i < n; ++i)
        out[i] = dec(in[i], dtype);
}
