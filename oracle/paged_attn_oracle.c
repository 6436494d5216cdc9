/*
 * CPU oracle for paged grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark may load this file's library. The product path
 * never calls it, and it shares no code, header or table with the HIP library.
 *
 * What it computes (written from the definitions, in double precision):
 *
 *   Paged cache (flashlet README, design bullets: the NHD pool
 *   [pages, page_size, kv_heads, head_dim]; the page table kv_indptr / kv_indices /
 *   last_page_len of a paged KV cache). Request r owns pages
 *   kv_indices[kv_indptr[r] .. kv_indptr[r+1]) and
 *       kv_len[r] = (kv_indptr[r+1] - kv_indptr[r] - 1) * page_size + last_page_len[r].
 *   Logical token t of request r sits in page kv_indices[kv_indptr[r] + t / page_size],
 *   slot t % page_size. The oracle first gathers each request's K and V rows into dense
 *   arrays, then works on the dense arrays only.
 *
 *   Ragged rows (flashlet README, design bullets: one plan()/run() call takes prefill
 *   chunks and decode rows together, and the causal mask covers both). Request r owns
 *   query rows qo_indptr[r] .. qo_indptr[r+1]. Reading of the causal mask: query row i
 *   of a request with qo_len rows sits at position kv_len - qo_len + i, so it attends
 *   keys t <= kv_len - qo_len + i (bottom-right alignment); for a single decode row this
 *   is every cached key.
 *
 *   Grouped-query heads (Torchlet README: GQA): query head h reads kv head
 *   h / (num_qo_heads / num_kv_heads).
 *
 *   Plain softmax attention per (row, head):
 *       s_t = scale * sum_d q[d] * k_t[d]
 *       m   = max_t s_t,  p_t = exp(s_t - m),  l = sum_t p_t
 *       out = sum_t p_t * v_t / l,  lse = m + log(l)          (natural log)
 *
 *   Split mode (num_splits > 1) follows "A library kernel for decode", What changed:
 *   a request's keys are cut into slices, each slice gives a partial result, and the
 *   partials are merged. Here the allowed keys [0, n) of a row are cut into num_splits
 *   consecutive slices of ceil(n / num_splits) keys (empty slices dropped); slice j gives
 *   (o_j, lse_j) by the plain formula above, and the merge is
 *       M = max_j lse_j,  w_j = exp(lse_j - M),  out = sum_j w_j o_j / sum_j w_j,
 *       lse = M + log(sum_j w_j).
 *   In exact arithmetic both modes give the same numbers.
 *
 * Storage types: 1 = IEEE binary16, 2 = bfloat16, 3 = binary32. 16-bit values are read
 * as raw bit patterns and decoded here by their published bit layouts.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARG (-1)
#define ORACLE_NO_MEM (-2)

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25);  /* (1024 + f) * 2^(e - 15 - 10) */
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
static double decode_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return (double)x;
}

static double load_elem(const void *base, int dtype, size_t i)
{
    switch (dtype) {
    case 1: return decode_f16(((const uint16_t *)base)[i]);
    case 2: return decode_bf16(((const uint16_t *)base)[i]);
    default: return (double)((const float *)base)[i];
    }
}

/* Decode n stored values to double (exported so the decoders can be checked alone). */
int oracle_decode(int dtype, const void *src, int64_t n, double *dst)
{
    if (dtype < 1 || dtype > 3 || n < 0 || (n > 0 && (!src || !dst)))
        return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < n; ++i)
        dst[i] = load_elem(src, dtype, (size_t)i);
    return ORACLE_OK;
}

/* Plain softmax attention of one query vector over keys [t0, t1) of dense K, V.
 * Writes o[D] (weighted mean) and returns lse; an empty range returns -inf, o = 0. */
static double attend_range(const double *qv, const double *K, const double *V, int D,
                           int t0, int t1, double scale, double *s, double *o)
{
    for (int d = 0; d < D; ++d)
        o[d] = 0.0;
    if (t1 <= t0)
        return -INFINITY;
    double m = -INFINITY;
    for (int t = t0; t < t1; ++t) {
        double acc = 0.0;
        const double *kt = K + (size_t)t * D;
        for (int d = 0; d < D; ++d)
            acc += qv[d] * kt[d];
        s[t] = scale * acc;
        if (s[t] > m)
            m = s[t];
    }
    double l = 0.0;
    for (int t = t0; t < t1; ++t) {
        double p = exp(s[t] - m);
        l += p;
        const double *vt = V + (size_t)t * D;
        for (int d = 0; d < D; ++d)
            o[d] += p * vt[d];
    }
    for (int d = 0; d < D; ++d)
        o[d] /= l;
    return m + log(l);
}

/*
 * out[rows * Hq * D] and lse[rows * Hq] (lse may be NULL) receive the unrounded
 * double results; rows = qo_indptr[batch] (qo_indptr == NULL means one row per request).
 * num_threads <= 0 uses the OpenMP default. Returns 0, or a negative code when the
 * metadata is inconsistent (no memory outside the given arrays is touched then).
 */
int oracle_paged_attention(int dtype, int batch, const int32_t *qo_indptr,
                           const int32_t *kv_indptr, const int32_t *kv_indices,
                           const int32_t *last_page_len, int64_t num_pages,
                           int num_qo_heads, int num_kv_heads, int head_dim, int page_size,
                           const void *q, const void *k_pool, const void *v_pool,
                           int causal, double sm_scale, int num_splits,
                           double *out, double *lse, int num_threads)
{
    if (dtype < 1 || dtype > 3 || batch < 0 || num_qo_heads <= 0 || num_kv_heads <= 0 ||
        num_qo_heads % num_kv_heads || head_dim <= 0 || page_size <= 0 || num_splits < 0)
        return ORACLE_BAD_ARG;
    if (batch == 0)
        return ORACLE_OK;
    if (!kv_indptr || !kv_indices || !last_page_len || !q || !k_pool || !v_pool || !out)
        return ORACLE_BAD_ARG;
    const int Hq = num_qo_heads, Hkv = num_kv_heads, D = head_dim, P = page_size;
    const int G = Hq / Hkv;
    if (kv_indptr[0] != 0 || (qo_indptr && qo_indptr[0] != 0))
        return ORACLE_BAD_ARG;
    for (int r = 0; r < batch; ++r) {
        int np_ = kv_indptr[r + 1] - kv_indptr[r];
        int qlen = qo_indptr ? qo_indptr[r + 1] - qo_indptr[r] : 1;
        if (np_ < 1 || qlen < 0 || last_page_len[r] < 1 || last_page_len[r] > P)
            return ORACLE_BAD_ARG;
        int64_t kv_len = (int64_t)(np_ - 1) * P + last_page_len[r];
        if (causal && qlen > kv_len)
            return ORACLE_BAD_ARG;
        for (int j = kv_indptr[r]; j < kv_indptr[r + 1]; ++j)
            if (kv_indices[j] < 0 || kv_indices[j] >= num_pages)
                return ORACLE_BAD_ARG;
    }
    const double scale = sm_scale > 0.0 ? sm_scale : 1.0 / sqrt((double)D);
    const int S = num_splits > 1 ? num_splits : 1;
    const int pairs = batch * Hkv;
    int status = ORACLE_OK;

#ifdef _OPENMP
    /* this call's thread count only; the process default stays as it was */
    const int nt = num_threads > 0 ? num_threads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#else
    (void)num_threads;
#endif
    for (int pr = 0; pr < pairs; ++pr) {
        const int r = pr / Hkv, g = pr % Hkv;
        const int np_ = kv_indptr[r + 1] - kv_indptr[r];
        const int kv_len = (np_ - 1) * P + last_page_len[r];
        const int row0 = qo_indptr ? qo_indptr[r] : r;
        const int qlen = qo_indptr ? qo_indptr[r + 1] - qo_indptr[r] : 1;
        double *K = malloc((size_t)kv_len * D * sizeof(double));
        double *V = malloc((size_t)kv_len * D * sizeof(double));
        double *s = malloc((size_t)kv_len * sizeof(double));
        double *qv = malloc((size_t)D * sizeof(double));
        double *o = malloc((size_t)D * sizeof(double));
        double *acc = malloc((size_t)D * sizeof(double));
        if (!K || !V || !s || !qv || !o || !acc) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = ORACLE_NO_MEM;
        } else {
            /* gather: token t -> page kv_indices[kv_indptr[r] + t / P], slot t % P */
            for (int t = 0; t < kv_len; ++t) {
                int64_t page = kv_indices[kv_indptr[r] + t / P];
                size_t src = (((size_t)page * P + (size_t)(t % P)) * Hkv + g) * D;
                for (int d = 0; d < D; ++d) {
                    K[(size_t)t * D + d] = load_elem(k_pool, dtype, src + d);
                    V[(size_t)t * D + d] = load_elem(v_pool, dtype, src + d);
                }
            }
            for (int i = 0; i < qlen; ++i) {
                const int n = causal ? kv_len - qlen + i + 1 : kv_len; /* keys [0, n) */
                for (int hh = 0; hh < G; ++hh) {
                    const int h = g * G + hh;
                    const size_t qi = ((size_t)(row0 + i) * Hq + h) * D;
                    for (int d = 0; d < D; ++d)
                        qv[d] = load_elem(q, dtype, qi + d);
                    double *dst = out + qi;
                    double L;
                    if (S == 1) {
                        L = attend_range(qv, K, V, D, 0, n, scale, s, dst);
                    } else {
                        const int len = (n + S - 1) / S;
                        double M = -INFINITY;
                        for (int j = 0; j < S; ++j) {
                            int a = j * len, b = a + len < n ? a + len : n;
                            if (a >= b)
                                continue;
                            double lj = attend_range(qv, K, V, D, a, b, scale, s, o);
                            if (lj > M)
                                M = lj;
                        }
                        double wsum = 0.0;
                        for (int d = 0; d < D; ++d)
                            acc[d] = 0.0;
                        for (int j = 0; j < S; ++j) {
                            int a = j * len, b = a + len < n ? a + len : n;
                            if (a >= b)
                                continue;
                            double lj = attend_range(qv, K, V, D, a, b, scale, s, o);
                            double w = exp(lj - M);
                            wsum += w;
                            for (int d = 0; d < D; ++d)
                                acc[d] += w * o[d];
                        }
                        for (int d = 0; d < D; ++d)
                            dst[d] = acc[d] / wsum;
                        L = M + log(wsum);
                    }
                    if (lse)
                        lse[(size_t)(row0 + i) * Hq + h] = L;
                }
            }
        }
        free(K);
        free(V);
        free(s);
        free(qv);
        free(o);
        free(acc);
    }
    return status;
}

/* Threads an OpenMP parallel region of the oracle uses (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Appending the new tokens' K/V to the paged cache (flashlet README, design bullets:
 * set_kv writes the step's new K and V rows into the NHD pool in place, before
 * attention reads it).
 *
 * Request r's query rows qo_indptr[r] .. qo_indptr[r+1] are its newest qo_len tokens,
 * so query row i of the request is logical token kv_len - qo_len + i (the same position
 * the bottom-right causal mask gives it). Its K row k_new[qo_indptr[r] + i, :, :]
 * (all kv heads, head_dim values each) is copied byte for byte into page
 * kv_indices[kv_indptr[r] + pos / P], slot pos % P of k_pool; likewise V. Nothing else
 * in the pools changes. Rows are copied as raw bytes (elem_bytes per value), so the
 * result is exact for every storage type.
 *
 * Returns 0, or a negative code (pools untouched) when the metadata is inconsistent:
 * a request with more new rows than cached tokens, or a page id outside the pool.
 */
int oracle_paged_kv_append(int elem_bytes, int batch, const int32_t *qo_indptr,
                           const int32_t *kv_indptr, const int32_t *kv_indices,
                           const int32_t *last_page_len, int64_t num_pages,
                           int num_kv_heads, int head_dim, int page_size,
                           const void *k_new, const void *v_new, void *k_pool, void *v_pool)
{
    if ((elem_bytes != 2 && elem_bytes != 4) || batch < 0 || num_kv_heads <= 0 ||
        head_dim <= 0 || page_size <= 0)
        return ORACLE_BAD_ARG;
    if (batch == 0)
        return ORACLE_OK;
    if (!kv_indptr || !kv_indices || !last_page_len || !k_pool || !v_pool)
        return ORACLE_BAD_ARG;
    if (kv_indptr[0] != 0 || (qo_indptr && qo_indptr[0] != 0))
        return ORACLE_BAD_ARG;
    const int P = page_size;
    const size_t token_bytes = (size_t)num_kv_heads * head_dim * elem_bytes;
    for (int r = 0; r < batch; ++r) {
        int np_ = kv_indptr[r + 1] - kv_indptr[r];
        int qlen = qo_indptr ? qo_indptr[r + 1] - qo_indptr[r] : 1;
        if (np_ < 1 || qlen < 0 || last_page_len[r] < 1 || last_page_len[r] > P)
            return ORACLE_BAD_ARG;
        int64_t kv_len = (int64_t)(np_ - 1) * P + last_page_len[r];
        if (qlen > kv_len)
            return ORACLE_BAD_ARG;
        if (qlen > 0 && (!k_new || !v_new))
            return ORACLE_BAD_ARG;
        for (int j = kv_indptr[r]; j < kv_indptr[r + 1]; ++j)
            if (kv_indices[j] < 0 || kv_indices[j] >= num_pages)
                return ORACLE_BAD_ARG;
    }
    for (int r = 0; r < batch; ++r) {
        const int np_ = kv_indptr[r + 1] - kv_indptr[r];
        const int kv_len = (np_ - 1) * P + last_page_len[r];
        const int row0 = qo_indptr ? qo_indptr[r] : r;
        const int qlen = qo_indptr ? qo_indptr[r + 1] - qo_indptr[r] : 1;
        for (int i = 0; i < qlen; ++i) {
            const int pos = kv_len - qlen + i;
            const int64_t page = kv_indices[kv_indptr[r] + pos / P];
            const size_t dst = ((size_t)page * P + (size_t)(pos % P)) * token_bytes;
            const size_t src = (size_t)(row0 + i) * token_bytes;
            memcpy((char *)k_pool + dst, (const char *)k_new + src, token_bytes);
            memcpy((char *)v_pool + dst, (const char *)v_new + src, token_bytes);
        }
    }
    return ORACLE_OK;
}

/*
 * Poisoning freed pages ("A library kernel for decode", closing paragraph: the engine's
 * gates poison pages when they return to the free list, so a kernel that still reads a
 * freed page produces NaN instead of stale numbers).
 *
 * Every element of each listed page (page_size * num_kv_heads * head_dim values, in
 * both pools) becomes the storage type's quiet NaN with a clear sign bit and a zero
 * payload: binary16 0x7E00, bfloat16 0x7FC0, binary32 0x7FC00000. Other pages are not
 * touched; a page listed twice is poisoned once. v_pool may be NULL.
 * Returns 0, or a negative code (pools untouched) for a page id outside [0, num_pages).
 */
int oracle_paged_kv_poison(int dtype, int64_t page_elems, const int32_t *page_ids, int n,
                           int64_t num_pages, void *k_pool, void *v_pool)
{
    if (dtype < 1 || dtype > 3 || page_elems <= 0 || n < 0 || (n > 0 && (!page_ids || !k_pool)))
        return ORACLE_BAD_ARG;
    for (int j = 0; j < n; ++j)
        if (page_ids[j] < 0 || page_ids[j] >= num_pages)
            return ORACLE_BAD_ARG;
    for (int j = 0; j < n; ++j) {
        for (int pool = 0; pool < 2; ++pool) {
            void *base = pool ? v_pool : k_pool;
            if (!base)
                continue;
            const size_t first = (size_t)page_ids[j] * (size_t)page_elems;
            for (int64_t e = 0; e < page_elems; ++e) {
                if (dtype == 3)
                    ((uint32_t *)base)[first + (size_t)e] = 0x7FC00000u;
                else
                    ((uint16_t *)base)[first + (size_t)e] = dtype == 1 ? 0x7E00u : 0x7FC0u;
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Rotary position embedding (RoPE), for the KV append fused with RoPE.
 *
 * The pages name RoPE as one of the layers of the Qwen2.5-style decoder they run (Torchlet
 * README, the running example; flashlet README, roadmap: a RoPE fusion kernel) without
 * writing it out. Reading taken, the rotate-half form of that model family: a head vector
 * x of head_dim D pairs element i with element i + D/2 (i < D/2), and the pair turns by
 * the angle a_i = pos * f_i with f_i = theta^(-2i/D):
 *     y[i]       = x[i] cos(a_i) - x[i + D/2] sin(a_i)
 *     y[i + D/2] = x[i + D/2] cos(a_i) + x[i] sin(a_i)
 * Precision reading: f_i is rounded to binary32 and a_i is the binary32 product of
 * (float)pos and f_i, as model code builds its tables; cos, sin and the rotation are in
 * double. x holds rows x heads x D storage values, positions[r] is row r's position, and
 * y receives the rotated values in double.
 * Returns 0, or a negative code for bad arguments (odd head_dim, theta <= 0, ...).
 */
int oracle_rope(int dtype, int rows, int heads, int head_dim, const void *x,
                const int32_t *positions, double theta, double *y)
{
    if (dtype < 1 || dtype > 3 || rows < 0 || heads <= 0 || head_dim <= 0 || head_dim % 2 ||
        !(theta > 0.0))
        return ORACLE_BAD_ARG;
    if (rows > 0 && (!x || !positions || !y))
        return ORACLE_BAD_ARG;
    const int half = head_dim / 2;
    for (int r = 0; r < rows; ++r) {
        for (int h = 0; h < heads; ++h) {
            const size_t base = ((size_t)r * heads + h) * (size_t)head_dim;
            for (int i = 0; i < half; ++i) {
                const float f = (float)pow(theta, -2.0 * i / head_dim);
                const float a = (float)positions[r] * f;
                const double c = cos((double)a), s = sin((double)a);
                const size_t i1 = base + (size_t)i, i2 = base + (size_t)i + (size_t)half;
                const double x1 = load_elem(x, dtype, i1), x2 = load_elem(x, dtype, i2);
                y[i1] = x1 * c - x2 * s;
                y[i2] = x2 * c + x1 * s;
            }
        }
    }
    return ORACLE_OK;
}
