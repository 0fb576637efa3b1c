/*
 * fp64 CPU oracle for single-token decode attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or table with the HIP library and never calls it.
 *
 * What it computes, for every sequence b and query head h:
 *
 *   g      = h / (Hq / Hkv)                      query heads share KV heads in
 *                                                contiguous groups (GQA/MQA,
 *                                                "TensorRT-LLM加速大模型推理实战";
 *                                                "TensorRT-LLM 推理加速实战" 8.1)
 *   for t in [0, n_b):
 *     phys = block_tables[b][t / PS], slot = t % PS
 *                                                the page table lookup and page
 *                                                count of "TensorRT-LLM 深度实战",
 *                                                section 3.1
 *     s_t  = scale * sum_d q[b][h][d] * K[phys][g][slot][d]
 *   M = max_t s_t,  w_t = exp(s_t - M),  Z = sum_t w_t
 *   out[b][h][:] = sum_t w_t * V[phys][g][slot][:] / Z
 *                                                scaled dot-product scores, the
 *                                                max-subtracted softmax and the
 *                                                weighted sum of V of the fused
 *                                                attention kernel of
 *                                                "TensorRT-LLM 深度实战", 3.3
 *
 * Every stored input is decoded exactly into double (f16, bf16, int8 x fp32
 * scale and fp8 e4m3 x fp32 scale are all exact in fp64) and all arithmetic is fp64.  A sequence with
 * n_b == 0 yields zeros.  Where the pages are silent the readings are: pool
 * layout [page][kv_head][slot][dim], contiguous GQA groups, context length
 * counting every cached token, int8 value = scale * code, fp8 value =
 * scale * e4m3(code).
 *
 * Compiled with -ffp-contract=off so every product and sum rounds as written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F16 = 0, ORC_BF16 = 1, ORC_I8 = 2, ORC_FP8 = 3 };
enum { ORC_OK = 0, ORC_BAD_ARG = -1, ORC_BAD_PAGE = -2, ORC_NO_MEM = -3 };

/* IEEE 754 binary16 -> double, exact (normals, subnormals, inf, nan). */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* 0.m * 2^-14 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);    /* 1.m * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 -> double, exact: bf16 is the top half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* FP8 E4M3 as the OCP 8-bit floating point specification defines it (the
 * "e4m3fn" encoding): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent field 0 holds subnormals 0.m * 2^-6; S.1111.111 is NaN;
 * there are no infinities, so the largest magnitude is 1.75 * 2^8 = 448.
 * Exact in double. */
double oracle_fp8e4m3_to_f64(uint8_t b)
{
    int sign = b >> 7;
    int e = (b >> 3) & 0xf;
    int m = b & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);                  /* 0.m * 2^-6 */
    else
        v = ldexp((double)(m | 8), e - 10);        /* 1.m * 2^(e-7) */
    return sign ? -v : v;
}

static double load_elem(int dtype, const void *base, size_t idx)
{
    if (dtype == ORC_F16)
        return oracle_f16_to_f64(((const uint16_t *)base)[idx]);
    if (dtype == ORC_BF16)
        return oracle_bf16_to_f64(((const uint16_t *)base)[idx]);
    if (dtype == ORC_FP8)
        return oracle_fp8e4m3_to_f64(((const uint8_t *)base)[idx]);
    return (double)((const int8_t *)base)[idx];
}

/* KV types stored with one fp32 scale per token per KV head. */
static int scaled_kv(int dtype) { return dtype == ORC_I8 || dtype == ORC_FP8; }

typedef struct {
    int B, Hq, Hkv, D, PS;
    int q_dtype, kv_dtype;
    const void *q;
    const void *k_pages, *v_pages;
    const float *k_scale, *v_scale;
    const int32_t *page_index;
    int num_pages, n_host_pages;
    const int32_t *block_tables;
    int max_blocks;
    const int32_t *context_lens;
    double scale;
} problem;

/* Host row of the page holding token t of sequence b, or -1 if the block
 * table entry does not name a stored page. */
static long page_row(const problem *p, int b, int t)
{
    int j = t / p->PS;
    if (j >= p->max_blocks)
        return -1;
    int phys = p->block_tables[(size_t)b * p->max_blocks + j];
    if (phys < 0 || phys >= p->num_pages)
        return -1;
    long row = p->page_index ? p->page_index[phys] : phys;
    if (row < 0 || row >= p->n_host_pages)
        return -1;
    return row;
}

/* K (which = 0) or V (which = 1) element d of token t, sequence b, kv head g. */
static double kv_elem(const problem *p, int which, long row, int g, int slot, int d)
{
    size_t tile = ((size_t)row * p->Hkv + g) * p->PS + slot;
    const void *base = which ? p->v_pages : p->k_pages;
    double x = load_elem(p->kv_dtype, base, tile * p->D + d);
    if (scaled_kv(p->kv_dtype)) {
        const float *sc = which ? p->v_scale : p->k_scale;
        x = (double)sc[tile] * x;
    }
    return x;
}

/* Scores s_t = scale * <q, k_t> for the query vector at element offset qoff
 * of q, against the keys of kv head g of sequence b, t in [t0, t1); returns
 * 0 or ORC_BAD_PAGE. */
static int scores_q(const problem *p, size_t qoff, int g, int b, int t0, int t1, double *s)
{
    for (int t = t0; t < t1; ++t) {
        long row = page_row(p, b, t);
        if (row < 0)
            return ORC_BAD_PAGE;
        double dot = 0.0;
        for (int d = 0; d < p->D; ++d)
            dot += load_elem(p->q_dtype, p->q, qoff + d) * kv_elem(p, 0, row, g, t % p->PS, d);
        s[t - t0] = p->scale * dot;
    }
    return ORC_OK;
}

/* Decode: the query of sequence b, head h is row b of q [B][Hq][D]. */
static int scores(const problem *p, int b, int h, int t0, int t1, double *s)
{
    int g = h / (p->Hq / p->Hkv);
    size_t qoff = ((size_t)b * p->Hq + h) * p->D;
    return scores_q(p, qoff, g, b, t0, t1, s);
}

/* Softmax-weighted sum over tokens [t0, t1) against a given max M:
 * writes acc[d] = sum_t exp(s_t - M) * v_t[d] and returns sum_t exp(s_t - M). */
static double weighted_v_g(const problem *p, int g, int b, int t0, int t1,
                           const double *s, double M, double *acc)
{
    for (int d = 0; d < p->D; ++d)
        acc[d] = 0.0;
    double Z = 0.0;
    for (int t = t0; t < t1; ++t) {
        long row = page_row(p, b, t);
        double w = exp(s[t - t0] - M);
        Z += w;
        for (int d = 0; d < p->D; ++d)
            acc[d] += w * kv_elem(p, 1, row, g, t % p->PS, d);
    }
    return Z;
}

static double weighted_v(const problem *p, int b, int h, int t0, int t1,
                         const double *s, double M, double *acc)
{
    int g = h / (p->Hq / p->Hkv);
    return weighted_v_g(p, g, b, t0, t1, s, M, acc);
}

static int check(const problem *p)
{
    if (p->B < 0 || p->Hq <= 0 || p->Hkv <= 0 || p->D <= 0 || p->PS <= 0)
        return ORC_BAD_ARG;
    if (p->Hq % p->Hkv)
        return ORC_BAD_ARG;
    if (scaled_kv(p->kv_dtype) && (!p->k_scale || !p->v_scale))
        return ORC_BAD_ARG;
    return ORC_OK;
}

/*
 * out[B][Hq][D] (double).  Pools hold n_host_pages pages laid out
 * [page][Hkv][PS][D]; page_index (length num_pages, may be NULL for identity)
 * maps a physical page id from the block table to its host row.
 */
int oracle_paged_decode(int B, int Hq, int Hkv, int D, int PS,
                        int q_dtype, const void *q,
                        int kv_dtype, const void *k_pages, const void *v_pages,
                        const float *k_scale, const float *v_scale,
                        const int32_t *page_index, int num_pages, int n_host_pages,
                        const int32_t *block_tables, int max_blocks,
                        const int32_t *context_lens, float scale,
                        double *out, int n_threads)
{
    problem p = {B, Hq, Hkv, D, PS, q_dtype, kv_dtype, q, k_pages, v_pages,
                 k_scale, v_scale, page_index, num_pages, n_host_pages,
                 block_tables, max_blocks, context_lens, (double)scale};
    int rc = check(&p);
    if (rc)
        return rc;
    int status = ORC_OK;
    long units = (long)B * Hq;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (long u = 0; u < units; ++u) {
        int b = (int)(u / Hq), h = (int)(u % Hq);
        int n = context_lens[b];
        double *o = out + (size_t)u * D;
        if (n <= 0) {
            for (int d = 0; d < D; ++d)
                o[d] = 0.0;
            continue;
        }
        double *s = (double *)malloc(sizeof(double) * (size_t)n);
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        if (!s || !acc) {
#pragma omp atomic write
            status = ORC_NO_MEM;
            free(s);
            free(acc);
            continue;
        }
        if (scores(&p, b, h, 0, n, s) != ORC_OK) {
#pragma omp atomic write
            status = ORC_BAD_PAGE;
            for (int d = 0; d < D; ++d)
                o[d] = NAN;
        } else {
            double M = s[0];
            for (int t = 1; t < n; ++t)
                if (s[t] > M)
                    M = s[t];
            double Z = weighted_v(&p, b, h, 0, n, s, M, acc);
            for (int d = 0; d < D; ++d)
                o[d] = acc[d] / Z;
        }
        free(s);
        free(acc);
    }
    return status;
}

/*
 * The same attention computed over token partitions [k*T, (k+1)*T) and then
 * merged: per partition m_k = max s, l_k = sum exp(s - m_k),
 * o_k = sum exp(s - m_k) v; then M = max_k m_k, L = sum_k l_k exp(m_k - M),
 * out = sum_k o_k exp(m_k - M) / L.  Algebraically identical to
 * oracle_paged_decode; it exists to check that identity and, through the
 * optional stats outputs, the per-partition quantities themselves.
 *
 * part_m / part_l ([B][Hq][P]) and part_o ([B][Hq][P][D]) may be NULL; P is
 * ceil(max_context_len / T) where max_context_len is the largest entry of
 * context_lens.  Entries of partitions past a sequence's end are m = -inf,
 * l = 0, o = 0.
 */
int oracle_paged_decode_split(int B, int Hq, int Hkv, int D, int PS,
                              int q_dtype, const void *q,
                              int kv_dtype, const void *k_pages, const void *v_pages,
                              const float *k_scale, const float *v_scale,
                              const int32_t *page_index, int num_pages, int n_host_pages,
                              const int32_t *block_tables, int max_blocks,
                              const int32_t *context_lens, float scale,
                              int partition_tokens, int P,
                              double *part_m, double *part_l, double *part_o,
                              double *out, int n_threads)
{
    problem p = {B, Hq, Hkv, D, PS, q_dtype, kv_dtype, q, k_pages, v_pages,
                 k_scale, v_scale, page_index, num_pages, n_host_pages,
                 block_tables, max_blocks, context_lens, (double)scale};
    int rc = check(&p);
    if (rc)
        return rc;
    if (partition_tokens <= 0 || P < 0)
        return ORC_BAD_ARG;
    const int T = partition_tokens;
    int status = ORC_OK;
    long units = (long)B * Hq;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (long u = 0; u < units; ++u) {
        int b = (int)(u / Hq), h = (int)(u % Hq);
        int n = context_lens[b];
        int np_ = n > 0 ? (n + T - 1) / T : 0;
        double *o = out + (size_t)u * D;
        double *m = (double *)malloc(sizeof(double) * (size_t)(np_ > 0 ? np_ : 1));
        double *l = (double *)malloc(sizeof(double) * (size_t)(np_ > 0 ? np_ : 1));
        double *ok = (double *)malloc(sizeof(double) * (size_t)(np_ > 0 ? np_ : 1) * D);
        double *s = (double *)malloc(sizeof(double) * (size_t)T);
        if (!m || !l || !ok || !s || np_ > P) {
#pragma omp atomic write
            status = np_ > P ? ORC_BAD_ARG : ORC_NO_MEM;
            free(m); free(l); free(ok); free(s);
            continue;
        }
        int bad = 0;
        for (int k = 0; k < np_ && !bad; ++k) {
            int t0 = k * T, t1 = (k + 1) * T < n ? (k + 1) * T : n;
            if (scores(&p, b, h, t0, t1, s) != ORC_OK) {
                bad = 1;
                break;
            }
            double mk = s[0];
            for (int t = 1; t < t1 - t0; ++t)
                if (s[t] > mk)
                    mk = s[t];
            m[k] = mk;
            l[k] = weighted_v(&p, b, h, t0, t1, s, mk, ok + (size_t)k * D);
        }
        if (bad) {
#pragma omp atomic write
            status = ORC_BAD_PAGE;
            for (int d = 0; d < D; ++d)
                o[d] = NAN;
        } else if (np_ == 0) {
            for (int d = 0; d < D; ++d)
                o[d] = 0.0;
        } else {
            double M = m[0];
            for (int k = 1; k < np_; ++k)
                if (m[k] > M)
                    M = m[k];
            double L = 0.0;
            for (int k = 0; k < np_; ++k)
                L += l[k] * exp(m[k] - M);
            for (int d = 0; d < D; ++d) {
                double acc = 0.0;
                for (int k = 0; k < np_; ++k)
                    acc += ok[(size_t)k * D + d] * exp(m[k] - M);
                o[d] = acc / L;
            }
        }
        if (part_m || part_l || part_o) {
            for (int k = 0; k < P; ++k) {
                size_t idx = (size_t)u * P + k;
                int live = k < np_ && !bad;
                if (part_m) part_m[idx] = live ? m[k] : -INFINITY;
                if (part_l) part_l[idx] = live ? l[k] : 0.0;
                if (part_o)
                    for (int d = 0; d < D; ++d)
                        part_o[idx * D + d] = live ? ok[(size_t)k * D + d] : 0.0;
            }
        }
        free(m); free(l); free(ok); free(s);
    }
    return status;
}

/*
 * Chunked prefill (context attention over the paged cache).  Sequence b's
 * new tokens are query rows q_start[b] .. q_start[b+1]-1 of q [n_q][Hq][D]:
 * the last nq = q_start[b+1] - q_start[b] of the context_lens[b] tokens its
 * cache holds (their own K/V included).  Query i sits at position
 * context_lens[b] - nq + i and attends causally to keys 0 .. that position,
 * with the decode path's scaled-dot-product softmax.  out[n_q][Hq][D].
 */
int oracle_paged_prefill(int B, int Hq, int Hkv, int D, int PS,
                         int q_dtype, const void *q, const int32_t *q_start,
                         int kv_dtype, const void *k_pages, const void *v_pages,
                         const float *k_scale, const float *v_scale,
                         const int32_t *page_index, int num_pages, int n_host_pages,
                         const int32_t *block_tables, int max_blocks,
                         const int32_t *context_lens, float scale,
                         double *out, int n_threads)
{
    problem p = {B, Hq, Hkv, D, PS, q_dtype, kv_dtype, q, k_pages, v_pages,
                 k_scale, v_scale, page_index, num_pages, n_host_pages,
                 block_tables, max_blocks, context_lens, (double)scale};
    int rc = check(&p);
    if (rc)
        return rc;
    if (!q_start || q_start[0] != 0)
        return ORC_BAD_ARG;
    for (int b = 0; b < B; ++b) {
        int nq = q_start[b + 1] - q_start[b];
        if (nq < 0 || nq > context_lens[b])
            return ORC_BAD_ARG;
    }
    int status = ORC_OK;
    long units = (long)B * Hq;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (long u = 0; u < units; ++u) {
        int b = (int)(u / Hq), h = (int)(u % Hq);
        int g = h / (Hq / Hkv);
        int n = context_lens[b], nq = q_start[b + 1] - q_start[b];
        double *s = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        if (!s || !acc) {
#pragma omp atomic write
            status = ORC_NO_MEM;
            free(s);
            free(acc);
            continue;
        }
        for (int i = 0; i < nq; ++i) {
            long row = q_start[b] + i;
            int pos = n - nq + i;                 /* keys 0 .. pos */
            double *o = out + ((size_t)row * Hq + h) * D;
            if (scores_q(&p, ((size_t)row * Hq + h) * D, g, b, 0, pos + 1, s) != ORC_OK) {
#pragma omp atomic write
                status = ORC_BAD_PAGE;
                for (int d = 0; d < D; ++d)
                    o[d] = NAN;
                continue;
            }
            double M = s[0];
            for (int t = 1; t <= pos; ++t)
                if (s[t] > M)
                    M = s[t];
            double Z = weighted_v_g(&p, g, b, 0, pos + 1, s, M, acc);
            for (int d = 0; d < D; ++d)
                o[d] = acc[d] / Z;
        }
        free(s);
        free(acc);
    }
    return status;
}

/*
 * Scatter of appended tokens: token i of the batch goes to pool slot
 * slots[i] = page * PS + offset, i.e. row (page, kv head, offset) of each KV
 * head.  pool is [num_pages][Hkv][PS][row_bytes] bytes; src is
 * [n][Hkv][row_bytes].  Returns ORC_BAD_ARG for a slot outside the pool.
 */
int oracle_scatter_rows(int n, int Hkv, int PS, int num_pages, int row_bytes,
                        const int64_t *slots, const uint8_t *src, uint8_t *pool)
{
    for (int i = 0; i < n; ++i) {
        int64_t slot = slots[i];
        if (slot < 0 || slot >= (int64_t)num_pages * PS)
            return ORC_BAD_ARG;
        int64_t page = slot / PS, off = slot % PS;
        for (int g = 0; g < Hkv; ++g)
            memcpy(pool + (((size_t)page * Hkv + g) * PS + off) * row_bytes,
                   src + ((size_t)i * Hkv + g) * row_bytes, (size_t)row_bytes);
    }
    return ORC_OK;
}

/*
 * Quantisation of appended K/V rows, the encodings the readings fix for the
 * pages' int8 and FP8 KV caches: per row (one token of one KV head) of D
 * values, in fp32 arithmetic,
 *     s    = max(max_d |x_d|, 1e-5) / Q        (Q = 127 for int8, 448 for fp8)
 *     code = round-half-to-even(x_d / s)        (int8: clipped to [-127, 127];
 *                                                fp8: the nearest E4M3 value)
 * Codes are written as bytes ([n][D]), scales as fp32 ([n]).
 */

/* Nearest OCP E4M3 code to y, ties to even; magnitudes that round above
 * the largest finite value (448) give 448. */
uint8_t oracle_fp8e4m3_encode(float y)
{
    if (y != y)
        return 0x7f;
    uint8_t sign = signbit(y) ? 0x80 : 0;
    double a = fabs((double)y);
    if (a >= 464.0)                    /* at or past the midpoint above 448 */
        return sign | 0x7e;
    if (a < ldexp(1.0, -6)) {          /* subnormal range: multiples of 2^-9 */
        double m = rint(a * 512.0);    /* exact product; rint ties to even */
        return sign | (uint8_t)m;      /* m == 8 is the smallest normal, code 0x08 */
    }
    int e;
    frexp(a, &e);                      /* a = f * 2^e, f in [0.5, 1) */
    e -= 1;                            /* a = 1.x * 2^e */
    double m = rint((ldexp(a, -e) - 1.0) * 8.0);
    if (m == 8.0) {
        m = 0.0;
        e += 1;
    }
    int field = e + 7;
    if (field > 15 || (field == 15 && m == 7.0))
        return sign | 0x7e;
    return sign | (uint8_t)((field << 3) | (int)m);
}

int oracle_quantize_rows(int n, int D, int kind, const float *x, uint8_t *codes, float *scales)
{
    if (n < 0 || D <= 0 || (kind != ORC_I8 && kind != ORC_FP8))
        return ORC_BAD_ARG;
    const float qmax = kind == ORC_I8 ? 127.0f : 448.0f;
    for (int i = 0; i < n; ++i) {
        const float *row = x + (size_t)i * D;
        float amax = 0.0f;
        for (int d = 0; d < D; ++d)
            amax = fmaxf(amax, fabsf(row[d]));
        const float s = fmaxf(amax, 1e-5f) / qmax;
        scales[i] = s;
        for (int d = 0; d < D; ++d) {
            const float y = row[d] / s;
            uint8_t c;
            if (kind == ORC_I8) {
                float r = rintf(y);
                r = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
                c = (uint8_t)(int8_t)r;
            } else {
                c = oracle_fp8e4m3_encode(y);
            }
            codes[(size_t)i * D + d] = c;
        }
    }
    return ORC_OK;
}
