/*
 * kev_oracle.c -- plain fp64 CPU oracle for segment-isolated packed attention.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only tests/, the smoke check and
 * the bench's cpu_baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library and includes nothing from it.
 *
 * What it computes (written out as the plain definition, no tiling, no
 * online softmax, no reordering):
 *
 *   Inference-engine primer (sakurs2.com), section 2.1: causal self-attention
 *     Z = softmax(Q K^T / sqrt(d_h) + M) V,  M_ij = 0 if j <= i else -inf,
 *   with the softmax taken along each row.
 *
 *   Kev article (icman.com.cn), sections 2.1 and 2.3: several questions are
 *   packed into one token stream; question s occupies an interval of the
 *   stream and the mask is the AND of the causal mask and the block-diagonal
 *   isolation mask.  Intervals are read as half-open [cu[s], cu[s+1]), which
 *   is how the article's code slices them (start:end with end = start + len).
 *
 *   So for row i of segment [a, b), query head h and key/value head g:
 *     s_j   = (sum_c q[i,h,c] k[j,g,c]) / sqrt(d)        for a <= j <= i
 *     m     = max_j s_j
 *     w_j   = exp(s_j - m),  Z = sum_j w_j                (stable softmax,
 *                                                          primer section 2.4)
 *     out[i,h,c] = (sum_j w_j v[j,g,c]) / Z
 *   Positions where M = -inf are never visited, so their weight is exactly 0.
 *
 *   Grouped KV heads are not named on the pages; q head h reads KV head
 *   h / (heads / kv_heads), i.e. each KV head is logically repeated for a
 *   contiguous group of query heads (the KV-cache isolation article,
 *   hnwysp.cn, section 7.1, contrasts such a shared view with a copy).
 *
 *   Decode (primer section 2.2): the new query attends over the cached K/V
 *   plus the new token's K/V with no mask; the cache is written in place
 *   rather than concatenated.  Each request owns one fixed-capacity slot of
 *   a pre-allocated pool (Kev part 2, gsyq.cn, section 2.2).  The pool layout
 *   is [slot][K or V][kv head][position][d], the per-head cache
 *   [B, H, S_cache, d] of the isolation article's section 2.2 with slots in
 *   place of the batch.  cache_lens[r] counts the tokens in the slot after
 *   the append, so the sequence is pool rows 0..L-2 followed by k_new/v_new
 *   at position L-1.
 *
 * Inputs are the exact bits the GPU path sees (bf16 bits or fp32), widened
 * to double.  Outputs are double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BF16 0
#define ORACLE_F32 1

#define ORACLE_OK 0
#define ORACLE_BAD_ARG -1
#define ORACLE_BAD_SEQLENS -3
#define ORACLE_SLOT_OVERFLOW -4
#define ORACLE_BAD_SLOT -5
#define ORACLE_NO_MEMORY -7

static double widen(const void *base, int dtype, size_t idx)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static void put_threads(int n_threads)
{
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
}

int kev_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Plain softmax attention of one query vector over n key/value vectors.
 *   qv[d], kv[j*d + c], vv[j*d + c] (already widened), w[n] is scratch.
 *   out[c] = sum_j softmax_j(q.k_j / sqrt(d)) v_j[c]
 */
static void attend(const double *qv, const double *kv, const double *vv, int n, int d,
                   double *w, double *out)
{
    double scale = 1.0 / sqrt((double)d);
    double m = -INFINITY;
    for (int j = 0; j < n; j++) {
        double s = 0.0;
        for (int c = 0; c < d; c++)
            s += qv[c] * kv[(size_t)j * d + c];
        w[j] = s * scale;
        if (w[j] > m)
            m = w[j];
    }
    double z = 0.0;
    for (int j = 0; j < n; j++) {
        w[j] = exp(w[j] - m);
        z += w[j];
    }
    for (int c = 0; c < d; c++) {
        double acc = 0.0;
        for (int j = 0; j < n; j++)
            acc += w[j] * vv[(size_t)j * d + c];
        out[c] = acc / z;
    }
}

static int check_seqlens(const int32_t *cu, int32_t n_seg)
{
    if (n_seg < 0 || (n_seg > 0 && cu == NULL))
        return ORACLE_BAD_ARG;
    if (n_seg == 0)
        return ORACLE_OK;
    if (cu[0] != 0)
        return ORACLE_BAD_SEQLENS;
    for (int32_t s = 0; s < n_seg; s++)
        if (cu[s + 1] < cu[s])
            return ORACLE_BAD_SEQLENS;
    return ORACLE_OK;
}

static int check_heads(int32_t heads, int32_t kv_heads, int32_t d, int dtype)
{
    if (heads <= 0 || kv_heads <= 0 || d <= 0 || heads % kv_heads != 0)
        return ORACLE_BAD_ARG;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F32)
        return ORACLE_BAD_ARG;
    return ORACLE_OK;
}

/*
 * Output rows [i0, i1) of query head h, all inside segment [a, b).
 * Row i attends keys a..i of KV head h / G.  The segment's K and V for that
 * head are widened once (rows a..i1-1) and each row uses its causal prefix.
 */
static void segment_head(const void *q, const void *k, const void *v, int dtype,
                         int32_t a, int32_t i0, int32_t i1, int32_t h,
                         int32_t heads, int32_t kv_heads, int32_t d,
                         double *kbuf, double *vbuf, double *qv, double *w,
                         double *out /* rows i0..i1-1, [row][d] */)
{
    int32_t g = h / (heads / kv_heads);
    int32_t n = i1 - a;
    for (int32_t j = 0; j < n; j++)
        for (int32_t c = 0; c < d; c++) {
            size_t src = ((size_t)(a + j) * kv_heads + g) * d + c;
            kbuf[(size_t)j * d + c] = widen(k, dtype, src);
            vbuf[(size_t)j * d + c] = widen(v, dtype, src);
        }
    for (int32_t i = i0; i < i1; i++) {
        for (int32_t c = 0; c < d; c++)
            qv[c] = widen(q, dtype, ((size_t)i * heads + h) * d + c);
        attend(qv, kbuf, vbuf, i - a + 1, d, w, out + (size_t)(i - i0) * d);
    }
}

/*
 * Full packed prefill.
 *   q[T, heads, d], k/v[T, kv_heads, d] (bf16 bits or fp32), cu[n_seg+1].
 *   out[T, heads, d] double.  Threads take (segment, head) units.
 */
int kev_oracle_prefill(const void *q, const void *k, const void *v, int dtype,
                       const int32_t *cu, int32_t n_seg, int32_t heads, int32_t kv_heads,
                       int32_t d, double *out, int n_threads)
{
    int rc = check_seqlens(cu, n_seg);
    if (rc)
        return rc;
    rc = check_heads(heads, kv_heads, d, dtype);
    if (rc)
        return rc;
    if (n_seg == 0)
        return ORACLE_OK;
    int32_t maxlen = 0;
    for (int32_t s = 0; s < n_seg; s++)
        if (cu[s + 1] - cu[s] > maxlen)
            maxlen = cu[s + 1] - cu[s];
    long units = (long)n_seg * heads;
    int fail = 0;
    put_threads(n_threads);
#pragma omp parallel
    {
        double *kbuf = malloc(sizeof(double) * ((size_t)maxlen * d + 1));
        double *vbuf = malloc(sizeof(double) * ((size_t)maxlen * d + 1));
        double *seg_out = malloc(sizeof(double) * ((size_t)maxlen * d + 1));
        double *qv = malloc(sizeof(double) * d);
        double *w = malloc(sizeof(double) * ((size_t)maxlen + 1));
        if (!kbuf || !vbuf || !seg_out || !qv || !w) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long u = 0; u < units; u++) {
                int32_t s = (int32_t)(u / heads), h = (int32_t)(u % heads);
                int32_t a = cu[s], b = cu[s + 1];
                if (b == a)
                    continue;
                segment_head(q, k, v, dtype, a, a, b, h, heads, kv_heads, d,
                             kbuf, vbuf, qv, w, seg_out);
                for (int32_t i = a; i < b; i++)
                    memcpy(out + ((size_t)i * heads + h) * d, seg_out + (size_t)(i - a) * d,
                           sizeof(double) * d);
            }
        }
        free(kbuf);
        free(vbuf);
        free(seg_out);
        free(qv);
        free(w);
    }
    return fail ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Sampled outputs of the packed prefill: for each n, out_rows[n, :] is the
 * output of token rows[n] at query head row_heads[n].  Same arithmetic as
 * the full call; used where the full oracle would take too long.
 */
int kev_oracle_prefill_rows(const void *q, const void *k, const void *v, int dtype,
                            const int32_t *cu, int32_t n_seg, int32_t heads, int32_t kv_heads,
                            int32_t d, const int32_t *rows, const int32_t *row_heads,
                            int32_t n_rows, double *out_rows, int n_threads)
{
    int rc = check_seqlens(cu, n_seg);
    if (rc)
        return rc;
    rc = check_heads(heads, kv_heads, d, dtype);
    if (rc)
        return rc;
    int32_t T = n_seg > 0 ? cu[n_seg] : 0;
    for (int32_t n = 0; n < n_rows; n++)
        if (rows[n] < 0 || rows[n] >= T || row_heads[n] < 0 || row_heads[n] >= heads)
            return ORACLE_BAD_ARG;
    int fail = 0;
    put_threads(n_threads);
#pragma omp parallel
    {
        size_t cap = 0;
        double *kbuf = NULL, *vbuf = NULL, *w = NULL;
        double *qv = malloc(sizeof(double) * d);
        if (!qv) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int32_t n = 0; n < n_rows; n++) {
            if (!qv)
                continue;
            int32_t i = rows[n];
            /* the last segment s with cu[s] <= i; then cu[s+1] > i */
            int32_t lo = 0, hi = n_seg - 1;
            while (lo < hi) {
                int32_t mid = (lo + hi + 1) / 2;
                if (cu[mid] <= i)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            int32_t a = cu[lo];
            size_t need = (size_t)(i - a + 1);
            if (need > cap) {
                free(kbuf);
                free(vbuf);
                free(w);
                kbuf = malloc(sizeof(double) * need * d);
                vbuf = malloc(sizeof(double) * need * d);
                w = malloc(sizeof(double) * need);
                cap = need;
                if (!kbuf || !vbuf || !w) {
#pragma omp atomic write
                    fail = 1;
                    cap = 0;
                    continue;
                }
            }
            segment_head(q, k, v, dtype, a, i, i + 1, row_heads[n], heads, kv_heads, d,
                         kbuf, vbuf, qv, w, out_rows + (size_t)n * d);
        }
        free(kbuf);
        free(vbuf);
        free(w);
        free(qv);
    }
    return fail ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Single-token decode against the slot pool.
 *   q[n_req, heads, d], k_new/v_new[n_req, kv_heads, d],
 *   pool[n_slots][2][kv_heads][capacity][d], slot_ids[n_req], cache_lens[n_req].
 *   out[n_req, heads, d] double.
 * If pool_after is not NULL it receives a copy of the pool with row L-1 of
 * each request's slot replaced by k_new / v_new (the expected pool after
 * the in-place append); it must have the pool's size and element type.
 */
int kev_oracle_decode(const void *q, const void *pool, int32_t n_slots, int32_t capacity,
                      int32_t kv_heads, int32_t d, const int32_t *slot_ids,
                      const int32_t *cache_lens, const void *k_new, const void *v_new,
                      int32_t n_req, int32_t heads, int dtype, double *out, void *pool_after,
                      int n_threads)
{
    int rc = check_heads(heads, kv_heads, d, dtype);
    if (rc)
        return rc;
    if (n_req < 0 || n_slots <= 0 || capacity <= 0)
        return ORACLE_BAD_ARG;
    for (int32_t r = 0; r < n_req; r++) {
        if (slot_ids[r] < 0 || slot_ids[r] >= n_slots)
            return ORACLE_BAD_SLOT;
        if (cache_lens[r] < 1 || cache_lens[r] > capacity)
            return ORACLE_SLOT_OVERFLOW;
        for (int32_t r2 = 0; r2 < r; r2++)
            if (slot_ids[r2] == slot_ids[r])
                return ORACLE_BAD_SLOT;
    }
    size_t esz = dtype == ORACLE_F32 ? 4 : 2;
    size_t plane = (size_t)capacity * d;                 /* one (slot, K|V, head) */
    size_t slot_elems = (size_t)2 * kv_heads * plane;
    int G = heads / kv_heads;
    long units = (long)n_req * heads;
    int fail = 0;
    put_threads(n_threads);
#pragma omp parallel
    {
        double *kbuf = malloc(sizeof(double) * plane);
        double *vbuf = malloc(sizeof(double) * plane);
        double *qv = malloc(sizeof(double) * d);
        double *w = malloc(sizeof(double) * capacity);
        if (!kbuf || !vbuf || !qv || !w) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long u = 0; u < units; u++) {
                int32_t r = (int32_t)(u / heads), h = (int32_t)(u % heads), g = h / G;
                int32_t L = cache_lens[r];
                size_t kbase = (size_t)slot_ids[r] * slot_elems + (size_t)g * plane;
                size_t vbase = kbase + (size_t)kv_heads * plane;
                for (int32_t j = 0; j < L - 1; j++)
                    for (int32_t c = 0; c < d; c++) {
                        kbuf[(size_t)j * d + c] = widen(pool, dtype, kbase + (size_t)j * d + c);
                        vbuf[(size_t)j * d + c] = widen(pool, dtype, vbase + (size_t)j * d + c);
                    }
                for (int32_t c = 0; c < d; c++) {
                    size_t src = ((size_t)r * kv_heads + g) * d + c;
                    kbuf[(size_t)(L - 1) * d + c] = widen(k_new, dtype, src);
                    vbuf[(size_t)(L - 1) * d + c] = widen(v_new, dtype, src);
                    qv[c] = widen(q, dtype, ((size_t)r * heads + h) * d + c);
                }
                attend(qv, kbuf, vbuf, L, d, w, out + ((size_t)r * heads + h) * d);
            }
        }
        free(kbuf);
        free(vbuf);
        free(qv);
        free(w);
    }
    if (fail)
        return ORACLE_NO_MEMORY;
    if (pool_after) {
        memcpy(pool_after, pool, esz * slot_elems * (size_t)n_slots);
        for (int32_t r = 0; r < n_req; r++)
            for (int32_t g = 0; g < kv_heads; g++) {
                size_t kdst = (size_t)slot_ids[r] * slot_elems + (size_t)g * plane +
                              (size_t)(cache_lens[r] - 1) * d;
                size_t vdst = kdst + (size_t)kv_heads * plane;
                size_t src = ((size_t)r * kv_heads + g) * d;
                memcpy((char *)pool_after + kdst * esz, (const char *)k_new + src * esz, esz * d);
                memcpy((char *)pool_after + vdst * esz, (const char *)v_new + src * esz, esz * d);
            }
    }
    return ORACLE_OK;
}

/*
 * Prefill-to-slot handoff: question s of a packed prefill gets slot slot_ids[s]
 * on entry, and its K/V rows become rows 0..len-1 of that slot, written in
 * place (Kev part 2, gsyq.cn, section 2.2: one slot per question, assigned on
 * entry; primer, sakurs2.com, section 2.2: the cache is pre-allocated space
 * written in place, not concatenated).
 *   k/v[T, kv_heads, d] with T = cu[n_seg]; pool[n_slots][2][kv_heads][capacity][d].
 *   pool_after receives a copy of the pool with those rows replaced; every
 *   other row keeps its bytes.
 */
int kev_oracle_store_kv(const void *k, const void *v, int dtype, const int32_t *cu,
                        int32_t n_seg, int32_t kv_heads, int32_t d, const int32_t *slot_ids,
                        const void *pool, int32_t n_slots, int32_t capacity, void *pool_after)
{
    int rc = check_seqlens(cu, n_seg);
    if (rc)
        return rc;
    if (kv_heads <= 0 || d <= 0 || n_slots <= 0 || capacity <= 0 ||
        (dtype != ORACLE_BF16 && dtype != ORACLE_F32))
        return ORACLE_BAD_ARG;
    for (int32_t s = 0; s < n_seg; s++) {
        if (slot_ids[s] < 0 || slot_ids[s] >= n_slots)
            return ORACLE_BAD_SLOT;
        if (cu[s + 1] - cu[s] > capacity)
            return ORACLE_SLOT_OVERFLOW;
        for (int32_t s2 = 0; s2 < s; s2++)
            if (slot_ids[s2] == slot_ids[s])
                return ORACLE_BAD_SLOT;
    }
    size_t esz = dtype == ORACLE_F32 ? 4 : 2;
    size_t plane = (size_t)capacity * d;
    size_t slot_elems = (size_t)2 * kv_heads * plane;
    memcpy(pool_after, pool, esz * slot_elems * (size_t)n_slots);
    for (int32_t s = 0; s < n_seg; s++)
        for (int32_t i = cu[s]; i < cu[s + 1]; i++)
            for (int32_t g = 0; g < kv_heads; g++) {
                size_t kdst = (size_t)slot_ids[s] * slot_elems + (size_t)g * plane +
                              (size_t)(i - cu[s]) * d;
                size_t vdst = kdst + (size_t)kv_heads * plane;
                size_t src = ((size_t)i * kv_heads + g) * d;
                memcpy((char *)pool_after + kdst * esz, (const char *)k + src * esz, esz * d);
                memcpy((char *)pool_after + vdst * esz, (const char *)v + src * esz, esz * d);
            }
    return ORACLE_OK;
}

/*
 * Chunked prefill against a slot prefix: question s's new tokens [cu[s], cu[s+1])
 * continue the P = prefix_lens[s] rows already cached in slot slot_ids[s].  Query
 * row i of the chunk sits at position P + i of the question and attends to the
 * slot's rows 0..P-1 and the chunk's rows 0..i, i.e. the causal mask over the
 * concatenation (primer, sakurs2.com, sections 2.1 and 2.6: a new chunk's queries
 * see the cached prefix and their own causal block; Kev part 2, gsyq.cn, section
 * 2.2: the prefix lives in the question's slot).  The chunk's K/V rows are then
 * written in place as rows P..P+n-1 of the slot (pool_after; every other byte kept).
 *   q[T, heads, d], k/v[T, kv_heads, d], pool[n_slots][2][kv_heads][capacity][d];
 *   out[T, heads, d] double.
 */
int kev_oracle_chunked_prefill(const void *q, const void *k, const void *v, int dtype,
                               const int32_t *cu, int32_t n_seg, int32_t heads, int32_t kv_heads,
                               int32_t d, const int32_t *slot_ids, const int32_t *prefix_lens,
                               const void *pool, int32_t n_slots, int32_t capacity, double *out,
                               void *pool_after, int n_threads)
{
    int rc = check_seqlens(cu, n_seg);
    if (rc)
        return rc;
    rc = check_heads(heads, kv_heads, d, dtype);
    if (rc)
        return rc;
    if (n_slots <= 0 || capacity <= 0)
        return ORACLE_BAD_ARG;
    for (int32_t s = 0; s < n_seg; s++) {
        if (slot_ids[s] < 0 || slot_ids[s] >= n_slots)
            return ORACLE_BAD_SLOT;
        if (prefix_lens[s] < 0 || prefix_lens[s] + (cu[s + 1] - cu[s]) > capacity)
            return ORACLE_SLOT_OVERFLOW;
        for (int32_t s2 = 0; s2 < s; s2++)
            if (slot_ids[s2] == slot_ids[s])
                return ORACLE_BAD_SLOT;
    }
    size_t esz = dtype == ORACLE_F32 ? 4 : 2;
    size_t plane = (size_t)capacity * d;
    size_t slot_elems = (size_t)2 * kv_heads * plane;
    int G = heads / kv_heads;
    long units = (long)n_seg * heads;
    int fail = 0;
    put_threads(n_threads);
#pragma omp parallel
    {
        double *kbuf = malloc(sizeof(double) * plane);
        double *vbuf = malloc(sizeof(double) * plane);
        double *qv = malloc(sizeof(double) * d);
        double *w = malloc(sizeof(double) * capacity);
        if (!kbuf || !vbuf || !qv || !w) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic)
            for (long u = 0; u < units; u++) {
                int32_t s = (int32_t)(u / heads), h = (int32_t)(u % heads), g = h / G;
                int32_t a = cu[s], n = cu[s + 1] - cu[s], P = prefix_lens[s];
                size_t kbase = (size_t)slot_ids[s] * slot_elems + (size_t)g * plane;
                size_t vbase = (size_t)slot_ids[s] * slot_elems + (size_t)(kv_heads + g) * plane;
                /* keys 0..P-1 from the slot, P..P+n-1 from the chunk */
                for (size_t e = 0; e < (size_t)P * d; e++) {
                    kbuf[e] = widen(pool, dtype, kbase + e);
                    vbuf[e] = widen(pool, dtype, vbase + e);
                }
                for (int32_t j = 0; j < n; j++)
                    for (int32_t c = 0; c < d; c++) {
                        size_t src = ((size_t)(a + j) * kv_heads + g) * d + c;
                        kbuf[(size_t)(P + j) * d + c] = widen(k, dtype, src);
                        vbuf[(size_t)(P + j) * d + c] = widen(v, dtype, src);
                    }
                for (int32_t i = 0; i < n; i++) {
                    for (int32_t c = 0; c < d; c++)
                        qv[c] = widen(q, dtype, ((size_t)(a + i) * heads + h) * d + c);
                    attend(qv, kbuf, vbuf, P + i + 1, d, w, out + ((size_t)(a + i) * heads + h) * d);
                }
            }
        }
        free(kbuf);
        free(vbuf);
        free(qv);
        free(w);
    }
    if (fail)
        return ORACLE_NO_MEMORY;
    if (pool_after) {
        memcpy(pool_after, pool, esz * slot_elems * (size_t)n_slots);
        for (int32_t s = 0; s < n_seg; s++)
            for (int32_t i = cu[s]; i < cu[s + 1]; i++)
                for (int32_t g = 0; g < kv_heads; g++) {
                    /* element offsets of the K row and the V row P + (i - cu[s]) of head g */
                    size_t row = (size_t)(prefix_lens[s] + i - cu[s]);
                    size_t to_k = ((size_t)slot_ids[s] * 2 * kv_heads + g) * plane + row * d;
                    size_t to_v = ((size_t)slot_ids[s] * 2 * kv_heads + kv_heads + g) * plane + row * d;
                    size_t from = ((size_t)i * kv_heads + g) * d;
                    memcpy((char *)pool_after + to_k * esz, (const char *)k + from * esz, esz * d);
                    memcpy((char *)pool_after + to_v * esz, (const char *)v + from * esz, esz * d);
                }
    }
    return ORACLE_OK;
}

/*
 * Decode against a paged KV pool (primer, sakurs2.com, section 2.5): the cache is cut into
 * fixed-size blocks of `block_size` positions that can sit anywhere in the pool, and request
 * r finds its position p in block block_tables[r][p / block_size], row p % block_size.  Apart
 * from where the rows live, the step is the slot decode above: the new K/V row is written in
 * place at position L-1 (section 2.2), and the query attends over positions 0..L-1.
 *   pool[n_blocks][2][kv_heads][block_size][d]; block_tables[n_req][max_blocks];
 *   positions 0..L-2 are read before any append of the call.  Blocks may be shared between
 *   requests for reading; an append target (block, row) must be touched by no other request.
 */
static int paged_row_taken(const int32_t *bt, int32_t max_blocks, const int32_t *lens, int32_t n_req,
                           int32_t bs, int32_t r, int32_t blk, int32_t row)
{
    for (int32_t r2 = 0; r2 < n_req; r2++) {
        if (r2 == r)
            continue;
        /* request r2 reads rows 0..L2-2 and writes row L2-1 */
        for (int32_t p = 0; p < lens[r2]; p++)
            if (bt[(size_t)r2 * max_blocks + p / bs] == blk && p % bs == row)
                return 1;
    }
    return 0;
}

int kev_oracle_paged_decode(const void *q, const void *pool, int32_t n_blocks, int32_t block_size,
                            int32_t kv_heads, int32_t d, const int32_t *block_tables, int32_t max_blocks,
                            const int32_t *cache_lens, const void *k_new, const void *v_new, int32_t n_req,
                            int32_t heads, int dtype, double *out, void *pool_after, int n_threads)
{
    int rc = check_heads(heads, kv_heads, d, dtype);
    if (rc)
        return rc;
    if (n_req < 0 || n_blocks <= 0 || block_size <= 0 || max_blocks <= 0)
        return ORACLE_BAD_ARG;
    /* every length and block id first: the append check below walks other requests' rows */
    for (int32_t r = 0; r < n_req; r++) {
        int32_t L = cache_lens[r];
        if (L < 1 || (L - 1) / block_size >= max_blocks)
            return ORACLE_SLOT_OVERFLOW;
        for (int32_t j = 0; j <= (L - 1) / block_size; j++) {
            int32_t b = block_tables[(size_t)r * max_blocks + j];
            if (b < 0 || b >= n_blocks)
                return ORACLE_BAD_SLOT;
        }
    }
    for (int32_t r = 0; r < n_req; r++) {
        int32_t L = cache_lens[r];
        int32_t last = block_tables[(size_t)r * max_blocks + (L - 1) / block_size];
        if (paged_row_taken(block_tables, max_blocks, cache_lens, n_req, block_size, r, last,
                            (L - 1) % block_size))
            return ORACLE_BAD_SLOT;
    }
    size_t esz = dtype == ORACLE_F32 ? 4 : 2;
    size_t head_rows = (size_t)block_size * d;              /* one (block, K|V, head) */
    size_t block_elems = (size_t)2 * kv_heads * head_rows;
    int32_t cap = max_blocks * block_size;
    int G = heads / kv_heads;
    long units = (long)n_req * heads;
    int fail = 0;
    put_threads(n_threads);
#pragma omp parallel
    {
        double *kbuf = malloc(sizeof(double) * (size_t)cap * d);
        double *vbuf = malloc(sizeof(double) * (size_t)cap * d);
        double *qv = malloc(sizeof(double) * d);
        double *w = malloc(sizeof(double) * cap);
        if (!kbuf || !vbuf || !qv || !w) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long u = 0; u < units; u++) {
                const int32_t r = (int32_t)(u / heads), h = (int32_t)(u % heads);
                const int32_t g = h / G;
                int32_t L = cache_lens[r];
                const int32_t *table = block_tables + (size_t)r * max_blocks;
                for (int32_t p = 0; p < L - 1; p++) {
                    size_t at = (size_t)table[p / block_size] * block_elems + (size_t)g * head_rows +
                                (size_t)(p % block_size) * d;
                    for (int32_t c = 0; c < d; c++) {
                        kbuf[(size_t)p * d + c] = widen(pool, dtype, at + c);
                        vbuf[(size_t)p * d + c] = widen(pool, dtype, at + (size_t)kv_heads * head_rows + c);
                    }
                }
                for (int32_t c = 0; c < d; c++) {
                    size_t src = ((size_t)r * kv_heads + g) * d + c, last = (size_t)(L - 1) * d + c;
                    kbuf[last] = widen(k_new, dtype, src);
                    vbuf[last] = widen(v_new, dtype, src);
                    qv[c] = widen(q, dtype, ((size_t)r * heads + h) * d + c);
                }
                attend(qv, kbuf, vbuf, L, d, w, out + ((size_t)r * heads + h) * d);
            }
        }
        free(kbuf);
        free(vbuf);
        free(qv);
        free(w);
    }
    if (fail)
        return ORACLE_NO_MEMORY;
    if (pool_after) {
        memcpy(pool_after, pool, esz * block_elems * (size_t)n_blocks);
        for (int32_t r = 0; r < n_req; r++) {
            int32_t p = cache_lens[r] - 1;
            int32_t blk = block_tables[(size_t)r * max_blocks + p / block_size];
            for (int32_t g = 0; g < kv_heads; g++) {
                size_t kat = (size_t)blk * block_elems + (size_t)g * head_rows + (size_t)(p % block_size) * d;
                size_t vat = kat + (size_t)kv_heads * head_rows;
                size_t from = ((size_t)r * kv_heads + g) * d;
                memcpy((char *)pool_after + kat * esz, (const char *)k_new + from * esz, esz * d);
                memcpy((char *)pool_after + vat * esz, (const char *)v_new + from * esz, esz * d);
            }
        }
    }
    return ORACLE_OK;
}
