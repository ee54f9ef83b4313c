/*
 * oracle.c -- plain, slow, obviously correct CPU reference for paged
 * single-query decode attention, the INT8 symmetric KV quantizer and the
 * slot-mapped cache write.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library
 * and its Python binding) may include, link or call this file.  It shares no
 * header, constant, helper or table with the HIP sources; dtype codes below
 * are defined here on their own.
 *
 * Sources (the four web pages on paged KV caches):
 *  - "Efficient AI Lecture 13: LLM deployment" notes (bittide.aicompass.dev
 *    mirror), section "PagedAttention", the four numbered steps: the cache of
 *    a sequence is cut into fixed-size logical blocks, physical blocks live
 *    anywhere in memory, and a block table translates logical block ids to
 *    physical ones.
 *  - docs.lazyllm.ai "Lesson 4: model deployment and inference acceleration",
 *    section 4.2 "PagedAttention": 16 tokens per block, per-request page
 *    table, global block pool, and the attention equation
 *    Attention(Q,K,V) = Softmax(Q K^T / sqrt(d)) V with Q of shape 1 x d and
 *    K, V of shape T x d; paging leaves that equation unchanged.
 *  - the same page, section 5.3 "KV Cache Quantization": symmetric INT8,
 *    K_q = round(K / s_K), s_K = max|K| / 127; the same section names FP8 as
 *    the alternative with a wider dynamic range, and the juejin page's
 *    "latest developments" list names FP8 KV caches in serving engines.
 *  - juejin.cn "LLM Engineer's Handbook -- inference optimization", the
 *    absmax-quantization passage with its worked example (0.1 with absmax 3.2
 *    gives code 4, dequantized 0.1008) and its PyTorch snippet that rounds
 *    with half-to-even rounding.
 *  - caojiahao2.github.io "LLM / MLLM inference", section 3.2, and the
 *    juejin page's "optimized attention" passage: online softmax keeps a
 *    running max and running sum; it is an exact rearrangement of the same
 *    softmax, so this oracle computes the plain definition instead.
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes of the repository):
 *  - 4-bit caches (caojiahao2 section 2.3 names INT4 KV quantization) take
 *    the linear b-bit formula of the lazyllm page, section 3.2, with b = 4
 *    over each (slot, kv head) row's own minimum and maximum;
 *  - one INT8 scale per (slot, kv head), separately for K and V; FP8 e4m3
 *    caches take the same per-row scale with 448 (the format's largest
 *    value) in place of 127;
 *  - quantizer form: s = fl32(amax / 127), code = clamp(rne(fl32(x / s)),
 *    -127, 127); amax == 0 gives s = 0 and all codes 0;
 *  - q head h reads kv head h / (Hq / Hkv) (contiguous GQA groups);
 *  - context_len == 0 gives an all-zero output row;
 *  - slot < 0 in a slot mapping means "skip this token".
 *
 * Everything floating point in the attention is done in IEEE double.  The
 * quantizer is done in IEEE single, because that is the precision the
 * reading above fixes for it.  Build: gcc -O2 -fopenmp -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Element type codes, defined here and only here.  OR_F8 is the 8-bit
 * floating-point format e4m3 (OCP "E4M3FN": sign, 4 exponent bits with bias
 * 7, 3 mantissa bits, no infinities, the all-ones exponent-and-mantissa
 * pattern is NaN, largest finite value 448). */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_I8 = 3, OR_F8 = 4, OR_U4 = 5 };
/* OR_U4: 4-bit codes 0..15, two per byte, element 2i in the low nibble of
 * byte i; each (slot, kv head) row carries two fp32 values (x_min, range). */

/* Scaled 8-bit caches: one fp32 scale per (slot, kv head). */
static int scaled(int dtype) { return dtype == OR_I8 || dtype == OR_F8; }

/* ------------------------------------------------------------------------ */
/* Exact widening of stored elements to double.                             */
/* ------------------------------------------------------------------------ */

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);             /* subnormal: frac * 2^-14 * 2^-10 */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25);  /* (1.frac) * 2^(expo-15) */
    }
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t b) {
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* e4m3 code -> value, from the format's definition. */
double oracle_f8_to_f64(uint8_t c) {
    int sign = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Nearest e4m3 code to x, ties to the even code (mantissa bit 0 clear).
 * Needs |x| <= 448 (callers clamp first).  Codes 0..126 hold the
 * non-negative finite values in increasing order; a binary search finds the
 * two neighbours of |x|. */
uint8_t oracle_f8_from_f32(float x) {
    const int neg = signbit(x) != 0;
    const double a = fabs((double)x);
    int lo = 0, hi = 126;                 /* invariant: value(lo) <= a */
    if (a >= oracle_f8_to_f64(126)) {
        lo = 126;
    } else {
        while (hi - lo > 1) {
            int mid = (lo + hi) / 2;
            if (oracle_f8_to_f64((uint8_t)mid) <= a) lo = mid; else hi = mid;
        }
        double dl = a - oracle_f8_to_f64((uint8_t)lo), dh = oracle_f8_to_f64((uint8_t)hi) - a;
        if (dh < dl || (dh == dl && (hi & 1) == 0)) lo = hi;
    }
    return (uint8_t)(lo | (neg ? 0x80 : 0));
}

static double elem(const void* base, size_t i, int dtype) {
    switch (dtype) {
    case OR_F32: return (double)((const float*)base)[i];
    case OR_F16: return oracle_f16_to_f64(((const uint16_t*)base)[i]);
    case OR_BF16: return oracle_bf16_to_f64(((const uint16_t*)base)[i]);
    case OR_I8: return (double)((const int8_t*)base)[i];
    case OR_F8: return oracle_f8_to_f64(((const uint8_t*)base)[i]);
    case OR_U4: {
        const uint8_t byte = ((const uint8_t*)base)[i / 2];
        return (double)((i % 2) ? (byte >> 4) : (byte & 15));
    }
    default: return NAN;
    }
}

static size_t elem_size(int dtype) {
    return dtype == OR_F32 ? 4 : (dtype == OR_I8 || dtype == OR_F8 ? 1 : 2);
}

/* ------------------------------------------------------------------------ */
/* Gather (paging) + dense attention for one (sequence, q head).            */
/* ------------------------------------------------------------------------ */

typedef struct {
    const void* q; int q_dtype;
    const void* k_cache; const void* v_cache; int cache_dtype;
    const float* k_scale; const float* v_scale;
    const int32_t* block_tables; int max_blocks_per_seq;
    const int32_t* context_lens;
    int B, Hq, Hkv, D, block_size, num_blocks;
    double scale;
} problem;

/* Logical token t of sequence b, kv head kvh -> element index of its first
 * channel in the pool [num_blocks][Hkv][block_size][D], and the index of its
 * per-token scale in [num_blocks][Hkv][block_size].  Returns -1 if the block
 * table names a block outside the pool. */
static long token_row(const problem* P, int b, int kvh, int t, long* scale_idx) {
    int logical = t / P->block_size;
    int offset = t % P->block_size;
    int32_t phys = P->block_tables[(size_t)b * P->max_blocks_per_seq + logical];
    if (phys < 0 || phys >= P->num_blocks) return -1;
    long row = ((long)phys * P->Hkv + kvh) * P->block_size + offset;
    *scale_idx = row;
    return row * P->D;
}

/* Gathered K and V of tokens [t0, t1) as dense double matrices. */
static int gather(const problem* P, int b, int kvh, int t0, int t1, double* K, double* V) {
    for (int t = t0; t < t1; ++t) {
        long si = 0;
        long base = token_row(P, b, kvh, t, &si);
        if (base < 0) return -1;
        double ks = 1.0, vs = 1.0;
        if (P->cache_dtype == OR_U4) {
            /* dequantization of the linear b-bit formula (b = 4):
             * x = x_min + code / (2^b - 1) * (x_max - x_min) */
            const double kmin = P->k_scale[2 * si], krange = P->k_scale[2 * si + 1];
            const double vmin = P->v_scale[2 * si], vrange = P->v_scale[2 * si + 1];
            for (int d = 0; d < P->D; ++d) {
                K[(size_t)(t - t0) * P->D + d] = kmin + elem(P->k_cache, base + d, OR_U4) / 15.0 * krange;
                V[(size_t)(t - t0) * P->D + d] = vmin + elem(P->v_cache, base + d, OR_U4) / 15.0 * vrange;
            }
            continue;
        }
        if (scaled(P->cache_dtype)) {
            ks = (double)P->k_scale[si];
            vs = (double)P->v_scale[si];
        }
        for (int d = 0; d < P->D; ++d) {
            K[(size_t)(t - t0) * P->D + d] = elem(P->k_cache, base + d, P->cache_dtype) * ks;
            V[(size_t)(t - t0) * P->D + d] = elem(P->v_cache, base + d, P->cache_dtype) * vs;
        }
    }
    return 0;
}

/* Softmax-weighted sum over tokens [t0, t1) of sequence b for q head h.
 * Outputs the max score m, the sum l of exp(s - m) and o = sum exp(s-m) V / l.
 * n == 0 gives m = -inf, l = 0, o = 0. */
static int attend_q(const problem* P, int b, int h, size_t qbase, int t0, int t1, double* m_out,
                    double* l_out, double* o);

static int attend(const problem* P, int b, int h, int t0, int t1, double* m_out, double* l_out,
                  double* o) {
    return attend_q(P, b, h, ((size_t)b * P->Hq + h) * P->D, t0, t1, m_out, l_out, o);
}

/* As attend, with the query vector at element qbase of P->q. */
static int attend_q(const problem* P, int b, int h, size_t qbase, int t0, int t1, double* m_out,
                    double* l_out, double* o) {
    int D = P->D;
    int g = P->Hq / P->Hkv;
    int kvh = h / g;
    int n = t1 - t0;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (n <= 0) { *m_out = -INFINITY; *l_out = 0.0; return 0; }

    double* K = malloc(sizeof(double) * (size_t)n * D);
    double* V = malloc(sizeof(double) * (size_t)n * D);
    double* s = malloc(sizeof(double) * (size_t)n);
    double* qv = malloc(sizeof(double) * (size_t)D);
    if (!K || !V || !s || !qv) { free(K); free(V); free(s); free(qv); return -2; }
    if (gather(P, b, kvh, t0, t1, K, V) != 0) { free(K); free(V); free(s); free(qv); return -1; }

    for (int d = 0; d < D; ++d) qv[d] = elem(P->q, qbase + d, P->q_dtype);

    /* scores s_t = scale * <q, K_t> */
    double m = -INFINITY;
    for (int t = 0; t < n; ++t) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qv[d] * K[(size_t)t * D + d];
        s[t] = P->scale * dot;
        if (s[t] > m) m = s[t];
    }
    /* softmax weights and weighted sum of V */
    double l = 0.0;
    for (int t = 0; t < n; ++t) {
        double w = exp(s[t] - m);
        l += w;
        for (int d = 0; d < D; ++d) o[d] += w * V[(size_t)t * D + d];
    }
    for (int d = 0; d < D; ++d) o[d] /= l;
    *m_out = m;
    *l_out = l;
    free(K); free(V); free(s); free(qv);
    return 0;
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Full decode attention.  out: double [B][Hq][D].  rows: optional list of
 * n_rows flattened (b * Hq + h) indices to compute; NULL computes all rows.
 * Rows not listed are left untouched.  window > 0 attends to the last
 * `window` positions only, [max(0, N - window), N): the sliding window of the
 * caojiahao2 page, section 2.3 (keep only the most recent window of the KV
 * cache); window == 0 attends to all N.  Returns 0, or a negative code when a
 * block table entry points outside the pool (-1) or memory ran out (-2). */
int oracle_paged_decode_window(double* out, const void* q, int q_dtype, const void* k_cache,
                               const void* v_cache, int cache_dtype, const float* k_scale,
                               const float* v_scale, const int32_t* block_tables,
                               int max_blocks_per_seq, const int32_t* context_lens, int B, int Hq,
                               int Hkv, int D, int block_size, int num_blocks, float scale,
                               int window, const int64_t* rows, long n_rows, int nthreads) {
    problem P = {q, q_dtype, k_cache, v_cache, cache_dtype, k_scale, v_scale, block_tables,
                 max_blocks_per_seq, context_lens, B, Hq, Hkv, D, block_size, num_blocks,
                 (double)scale};
    if (Hkv <= 0 || Hq % Hkv != 0 || block_size <= 0) return -3;
    long total = rows ? n_rows : (long)B * Hq;
    int status = 0;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < total; ++i) {
        long r = rows ? (long)rows[i] : i;
        int b = (int)(r / Hq), h = (int)(r % Hq);
        double m, l;
        int n = context_lens[b];
        int t0 = (window > 0 && n > window) ? n - window : 0;
        int rc = attend(&P, b, h, t0, n, &m, &l, out + (size_t)r * D);
        if (rc != 0) {
#pragma omp critical
            status = rc;
        }
    }
    return status;
}

int oracle_paged_decode(double* out, const void* q, int q_dtype, const void* k_cache,
                        const void* v_cache, int cache_dtype, const float* k_scale,
                        const float* v_scale, const int32_t* block_tables,
                        int max_blocks_per_seq, const int32_t* context_lens, int B, int Hq,
                        int Hkv, int D, int block_size, int num_blocks, float scale,
                        const int64_t* rows, long n_rows, int nthreads) {
    return oracle_paged_decode_window(out, q, q_dtype, k_cache, v_cache, cache_dtype, k_scale,
                                      v_scale, block_tables, max_blocks_per_seq, context_lens, B,
                                      Hq, Hkv, D, block_size, num_blocks, scale, 0, rows, n_rows,
                                      nthreads);
}

/* Attention for several query tokens per sequence over the paged cache: the
 * verification pass of speculative decoding, where the target model checks
 * k draft tokens in one forward pass (caojiahao2.github.io section 6;
 * lazyllm lesson 4, the speculative-decoding algorithm), or a prefill chunk.
 * Sequence b has N_b = context_lens[b] cached tokens, the last
 * q_len_b = query_start_loc[b + 1] - query_start_loc[b] of them being its
 * queries; query row r = query_start_loc[b] + j (j < q_len_b) sits at position
 * p = N_b - q_len_b + j and attends causally to positions 0..p.
 * q, out: [T][Hq][D] with T = query_start_loc[B].  A query with p < 0 (more
 * queries than tokens) gets a zero row. */
int oracle_paged_multi(double* out, const void* q, int q_dtype, const void* k_cache,
                       const void* v_cache, int cache_dtype, const float* k_scale,
                       const float* v_scale, const int32_t* block_tables,
                       int max_blocks_per_seq, const int32_t* context_lens,
                       const int32_t* query_start_loc, int B, int Hq, int Hkv, int D,
                       int block_size, int num_blocks, float scale, int nthreads) {
    problem P = {q, q_dtype, k_cache, v_cache, cache_dtype, k_scale, v_scale, block_tables,
                 max_blocks_per_seq, context_lens, B, Hq, Hkv, D, block_size, num_blocks,
                 (double)scale};
    if (Hkv <= 0 || Hq % Hkv != 0 || block_size <= 0) return -3;
    long T = query_start_loc[B];
    int status = 0;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < T * Hq; ++i) {
        long r = i / Hq;
        int h = (int)(i % Hq);
        int b = 0;
        while (b + 1 < B && query_start_loc[b + 1] <= r) ++b;
        int q_len = query_start_loc[b + 1] - query_start_loc[b];
        int p = context_lens[b] - q_len + (int)(r - query_start_loc[b]);
        double m, l;
        int rc = attend_q(&P, b, h, ((size_t)r * Hq + h) * D, 0, p + 1, &m, &l,
                          out + (size_t)i * D);
        if (rc != 0) {
#pragma omp critical
            status = rc;
        }
    }
    return status;
}

/* Split-context partials.  A context of N tokens is cut into
 * count = ceil(N / P) partitions (P = partition_size) of equal length, rounded
 * up to whole blocks: span = block_size * ceil(ceil(N / count) / block_size);
 * partition p holds tokens [p*span, min((p+1)*span, N)).  The pages fix no
 * split (the merge of running maxima and sums is exact whatever the split:
 * caojiahao2.github.io section 3.2), so this is a reading: the same number
 * of partitions as cutting at multiples of P, but of equal length, so that
 * no partition is a short stub.  The boundaries are pinned by hand-computed
 * spans in the tests; the final output does not depend on them.
 * m, l: double [B][Hq][NP]; o: double [B][Hq][NP][D].  Partitions with no
 * token get m = -inf, l = 0, o = 0.  The max score m is in natural-log units
 * of the score s = scale * <q, k>. */
int oracle_paged_partials(double* m_part, double* l_part, double* o_part, const void* q,
                          int q_dtype, const void* k_cache, const void* v_cache, int cache_dtype,
                          const float* k_scale, const float* v_scale,
                          const int32_t* block_tables, int max_blocks_per_seq,
                          const int32_t* context_lens, int B, int Hq, int Hkv, int D,
                          int block_size, int num_blocks, float scale, int partition_size,
                          int num_partitions, int nthreads) {
    problem P = {q, q_dtype, k_cache, v_cache, cache_dtype, k_scale, v_scale, block_tables,
                 max_blocks_per_seq, context_lens, B, Hq, Hkv, D, block_size, num_blocks,
                 (double)scale};
    if (Hkv <= 0 || Hq % Hkv != 0 || partition_size <= 0) return -3;
    long total = (long)B * Hq * num_partitions;
    int status = 0;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < total; ++i) {
        int p = (int)(i % num_partitions);
        long r = i / num_partitions;
        int b = (int)(r / Hq), h = (int)(r % Hq);
        int n = context_lens[b];
        int count = n > 0 ? (n + partition_size - 1) / partition_size : 0;
        int span = 0;
        if (count > 0) {
            int per = (n + count - 1) / count;
            span = (per + block_size - 1) / block_size * block_size;
        }
        int t0 = p < count ? p * span : n;
        int t1 = t0 + span < n ? t0 + span : n;
        int rc = attend(&P, b, h, t0, t1, m_part + i, l_part + i, o_part + (size_t)i * D);
        if (rc != 0) {
#pragma omp critical
            status = rc;
        }
    }
    return status;
}

/* Merge of partials: out = sum_p w_p o_p / sum_p w_p with w_p = l_p e^{m_p}
 * (computed relative to M = max_p m_p).  Partitions with l_p == 0 carry no
 * weight.  A row whose partitions are all empty gives 0. */
int oracle_merge_partials(double* out, const double* m_part, const double* l_part,
                          const double* o_part, long rows, int num_partitions, int D) {
    for (long r = 0; r < rows; ++r) {
        const double* m = m_part + r * num_partitions;
        const double* l = l_part + r * num_partitions;
        double M = -INFINITY;
        for (int p = 0; p < num_partitions; ++p)
            if (l[p] > 0.0 && m[p] > M) M = m[p];
        double* o = out + r * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (M == -INFINITY) continue;
        double wsum = 0.0;
        for (int p = 0; p < num_partitions; ++p) {
            if (!(l[p] > 0.0)) continue;
            double w = l[p] * exp(m[p] - M);
            wsum += w;
            for (int d = 0; d < D; ++d) o[d] += w * o_part[((size_t)r * num_partitions + p) * D + d];
        }
        for (int d = 0; d < D; ++d) o[d] /= wsum;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* INT8 symmetric quantization, one scale per row of D elements.            */
/* ------------------------------------------------------------------------ */

/* Widen one stored element to single precision.  Exact for f16/bf16/f32. */
static float elem_f32(const void* base, size_t i, int dtype) {
    return (float)elem(base, i, dtype);
}

/* Quantize one row: amax = max |x|; s = amax / 127 in single precision;
 * code = clamp(round-half-even(x / s), -127, 127) with the division in single
 * precision.  amax == 0 gives s = 0 and codes 0. */
static void quantize_row_i8(int8_t* codes, float* scale_out, const void* x, size_t base, int D,
                            int dtype) {
    float amax = 0.0f;
    for (int d = 0; d < D; ++d) {
        float a = fabsf(elem_f32(x, base + d, dtype));
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        *scale_out = 0.0f;
        for (int d = 0; d < D; ++d) codes[d] = 0;
        return;
    }
    volatile float s = amax / 127.0f;  /* one IEEE single-precision division */
    for (int d = 0; d < D; ++d) {
        volatile float r = elem_f32(x, base + d, dtype) / s;
        float c = nearbyintf(r);  /* default rounding mode: to nearest, ties to even */
        if (c > 127.0f) c = 127.0f;
        if (c < -127.0f) c = -127.0f;
        codes[d] = (int8_t)c;
    }
    *scale_out = s;
}

/* FP8 e4m3 row, same shape of rule with the format's largest value in place
 * of 127: s = amax / 448 in single precision; r = x / s in single precision,
 * clamped to [-448, 448] (it can exceed 448 by a rounding of s); code = the
 * nearest e4m3 value to r, ties to even.  amax == 0 gives s = 0 and codes 0. */
static void quantize_row_f8(uint8_t* codes, float* scale_out, const void* x, size_t base, int D,
                            int dtype) {
    float amax = 0.0f;
    for (int d = 0; d < D; ++d) {
        float a = fabsf(elem_f32(x, base + d, dtype));
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        *scale_out = 0.0f;
        for (int d = 0; d < D; ++d) codes[d] = 0;
        return;
    }
    volatile float s = amax / 448.0f;
    for (int d = 0; d < D; ++d) {
        volatile float r = elem_f32(x, base + d, dtype) / s;
        float c = r;
        if (c > 448.0f) c = 448.0f;
        if (c < -448.0f) c = -448.0f;
        codes[d] = oracle_f8_from_f32(c);
    }
    *scale_out = s;
}

/* 4-bit row by the linear b-bit formula with b = 4, over the row's own
 * minimum and maximum: code = round((x - x_min) / (x_max - x_min) * 15),
 * evaluated left to right in single precision (x - x_min, then the division,
 * then the product), rounded half to even and clamped to [0, 15].
 * meta = (x_min, x_max - x_min); a constant row gives range 0 and codes 0.
 * codes: D / 2 bytes, element 2i in the low nibble of byte i. */
static void quantize_row_u4(uint8_t* codes, float* meta, const void* x, size_t base, int D,
                            int dtype) {
    float lo = elem_f32(x, base, dtype), hi = lo;
    for (int d = 1; d < D; ++d) {
        float v = elem_f32(x, base + d, dtype);
        if (v < lo) lo = v;
        if (v > hi) hi = v;
    }
    volatile float range = hi - lo;
    meta[0] = lo;
    meta[1] = range;
    for (int d = 0; d < D; d += 2) codes[d / 2] = 0;
    if (range == 0.0f) return;
    for (int d = 0; d < D; ++d) {
        volatile float diff = elem_f32(x, base + d, dtype) - lo;
        volatile float frac = diff / range;
        volatile float r = frac * 15.0f;
        float c = nearbyintf(r);
        if (c < 0.0f) c = 0.0f;
        if (c > 15.0f) c = 15.0f;
        codes[d / 2] |= (uint8_t)((int)c << (4 * (d % 2)));
    }
}

static void quantize_row(void* codes, float* scale_out, const void* x, size_t base, int D,
                         int dtype, int cache_dtype) {
    if (cache_dtype == OR_F8)
        quantize_row_f8((uint8_t*)codes, scale_out, x, base, D, dtype);
    else
        quantize_row_i8((int8_t*)codes, scale_out, x, base, D, dtype);
}

/* x: [rows][D] of dtype; codes: int8 [rows][D]; scales: float [rows]. */
int oracle_quantize_rows(int8_t* codes, float* scales, const void* x, int dtype, long rows, int D) {
    for (long r = 0; r < rows; ++r)
        quantize_row_i8(codes + (size_t)r * D, scales + r, x, (size_t)r * D, D, dtype);
    return 0;
}

/* 4-bit rows: codes uint8 [rows][D / 2], meta float [rows][2] = (x_min, range). */
int oracle_quantize_rows_u4(uint8_t* codes, float* meta, const void* x, int dtype, long rows,
                            int D) {
    if (D % 2) return -3;
    for (long r = 0; r < rows; ++r)
        quantize_row_u4(codes + (size_t)r * (D / 2), meta + 2 * r, x, (size_t)r * D, D, dtype);
    return 0;
}

/* As oracle_quantize_rows, to e4m3 codes (uint8 [rows][D]). */
int oracle_quantize_rows_f8(uint8_t* codes, float* scales, const void* x, int dtype, long rows,
                            int D) {
    for (long r = 0; r < rows; ++r)
        quantize_row_f8(codes + (size_t)r * D, scales + r, x, (size_t)r * D, D, dtype);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Slot-mapped cache write on host byte images of the pool.                 */
/* ------------------------------------------------------------------------ */

/* k, v: [T][Hkv][D] of src_dtype.  k_cache, v_cache: [num_blocks][Hkv][block_size][D]
 * of cache_dtype (equal to src_dtype, or OR_I8 / OR_F8).  k_scale, v_scale:
 * float [num_blocks][Hkv][block_size], used only for OR_I8 and OR_F8.  Token i with
 * slot = slot_mapping[i] >= 0 goes to block slot / block_size, offset
 * slot % block_size, for every kv head.  Negative slots are skipped.
 * Returns -1 if a slot is beyond the pool, -3 for an unsupported pairing. */
int oracle_kv_cache_write(const void* k, const void* v, void* k_cache, void* v_cache,
                          float* k_scale, float* v_scale, const int64_t* slot_mapping, long T,
                          int Hkv, int D, int block_size, int num_blocks, int src_dtype,
                          int cache_dtype) {
    if (cache_dtype != src_dtype && !scaled(cache_dtype) && cache_dtype != OR_U4) return -3;
    if (scaled(src_dtype) || src_dtype == OR_U4) return -3;
    size_t es = elem_size(cache_dtype);
    for (long i = 0; i < T; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0) continue;
        if (slot >= (int64_t)num_blocks * block_size) return -1;
        int64_t blk = slot / block_size, off = slot % block_size;
        for (int h = 0; h < Hkv; ++h) {
            size_t src = ((size_t)i * Hkv + h) * D;
            size_t dst_row = ((size_t)blk * Hkv + h) * block_size + (size_t)off;
            if (cache_dtype == OR_U4) {
                quantize_row_u4((uint8_t*)k_cache + dst_row * (D / 2), k_scale + 2 * dst_row, k,
                                src, D, src_dtype);
                quantize_row_u4((uint8_t*)v_cache + dst_row * (D / 2), v_scale + 2 * dst_row, v,
                                src, D, src_dtype);
            } else if (scaled(cache_dtype)) {
                quantize_row((int8_t*)k_cache + dst_row * D, k_scale + dst_row, k, src, D,
                             src_dtype, cache_dtype);
                quantize_row((int8_t*)v_cache + dst_row * D, v_scale + dst_row, v, src, D,
                             src_dtype, cache_dtype);
            } else {
                memcpy((char*)k_cache + dst_row * D * es, (const char*)k + src * es, D * es);
                memcpy((char*)v_cache + dst_row * D * es, (const char*)v + src * es, D * es);
            }
        }
    }
    return 0;
}

int oracle_num_threads(int nthreads) { return set_threads(nthreads); }
