/*
 * oracle_sanitize.c -- runs every entry point of oracle/kev_oracle.c on small inputs held in
 * exactly-sized heap buffers, built with AddressSanitizer and UndefinedBehaviorSanitizer, so
 * that an out-of-range read or write, or undefined arithmetic, anywhere in the oracle stops
 * the run.  Edge cases: empty and length-1 questions, grouped KV heads, decode at L = 1 and
 * L = capacity, a chunk with an empty prefix and one filling its slot, paged blocks of one
 * row, and every argument error the oracle reports.  A few results are also pinned: the
 * primer's worked example (section 2.4), a length-1 question returning its value row (the
 * mask leaves one key), and decode equal to the last row of a recompute (primer section 2.2).
 * Exit status 0 = every check passed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kev_oracle_prefill(const void *, const void *, const void *, int, const int32_t *, int32_t, int32_t,
                       int32_t, int32_t, double *, int);
int kev_oracle_prefill_rows(const void *, const void *, const void *, int, const int32_t *, int32_t,
                            int32_t, int32_t, int32_t, const int32_t *, const int32_t *, int32_t, double *,
                            int);
int kev_oracle_decode(const void *, const void *, int32_t, int32_t, int32_t, int32_t, const int32_t *,
                      const int32_t *, const void *, const void *, int32_t, int32_t, int, double *, void *,
                      int);
int kev_oracle_store_kv(const void *, const void *, int, const int32_t *, int32_t, int32_t, int32_t,
                        const int32_t *, const void *, int32_t, int32_t, void *);
int kev_oracle_chunked_prefill(const void *, const void *, const void *, int, const int32_t *, int32_t,
                               int32_t, int32_t, int32_t, const int32_t *, const int32_t *, const void *,
                               int32_t, int32_t, double *, void *, int);
int kev_oracle_paged_decode(const void *, const void *, int32_t, int32_t, int32_t, int32_t, const int32_t *,
                            int32_t, const int32_t *, const void *, const void *, int32_t, int32_t, int,
                            double *, void *, int);

static int failures = 0;
#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                  \
        }                                                                \
    } while (0)

static uint64_t rng_state = 88172645463325252ull;
static float frand(void)
{   /* xorshift64, uniform in [-2, 2) */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (float)((rng_state >> 11) * (1.0 / 9007199254740992.0)) * 4.0f - 2.0f;
}
static uint16_t bf16_bits(float x)
{   /* round to nearest even (inputs are finite) */
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static float *f32_buf(size_t n)
{
    float *p = malloc(n * sizeof *p);
    for (size_t i = 0; i < n; ++i) p[i] = frand();
    return p;
}
static uint16_t *bf16_buf(size_t n)
{
    uint16_t *p = malloc(n * sizeof *p);
    for (size_t i = 0; i < n; ++i) p[i] = bf16_bits(frand());
    return p;
}

static void prefill_cases(void)
{
    /* packed fp32 GQA prefill with empty and length-1 questions */
    const int32_t cu[] = {0, 5, 5, 6, 19, 19};
    const int32_t n_seg = 5, T = 19, H = 4, HK = 2, D = 8;
    float *q = f32_buf((size_t)T * H * D), *k = f32_buf((size_t)T * HK * D), *v = f32_buf((size_t)T * HK * D);
    double *out = malloc((size_t)T * H * D * sizeof(double));
    CHECK(kev_oracle_prefill(q, k, v, 1, cu, n_seg, H, HK, D, out, 0) == 0);
    for (int h = 0; h < H; ++h)   /* the length-1 question (row 5) returns its value row */
        for (int c = 0; c < D; ++c) CHECK(out[((size_t)5 * H + h) * D + c] == (double)v[((size_t)5 * HK + h / 2) * D + c]);
    /* sampled rows agree with the full call */
    const int32_t rows[] = {0, 4, 5, 18, 6};
    const int32_t rh[] = {0, 3, 1, 2, 3};
    double *orow = malloc(5 * D * sizeof(double));
    CHECK(kev_oracle_prefill_rows(q, k, v, 1, cu, n_seg, H, HK, D, rows, rh, 5, orow, 1) == 0);
    for (int i = 0; i < 5; ++i)
        for (int c = 0; c < D; ++c) CHECK(orow[i * D + c] == out[((size_t)rows[i] * H + rh[i]) * D + c]);
    /* argument errors */
    const int32_t bad_cu[] = {0, 7, 3};
    CHECK(kev_oracle_prefill(q, k, v, 1, bad_cu, 2, H, HK, D, out, 0) == -3);
    CHECK(kev_oracle_prefill(q, k, v, 1, cu, n_seg, 3, HK, D, out, 0) == -1);
    const int32_t bad_rows[] = {19};
    CHECK(kev_oracle_prefill_rows(q, k, v, 1, cu, n_seg, H, HK, D, bad_rows, rh, 1, orow, 0) != 0);
    free(q), free(k), free(v), free(out), free(orow);

    /* the primer's worked example: scores 1..4 against values 10..40 (d = 16, q = [4,0,..]) */
    const int32_t cu4[] = {0, 4};
    float q4[4 * 16] = {0}, k4[4 * 16] = {0}, v4[4 * 16] = {0};
    for (int j = 0; j < 4; ++j) {
        q4[j * 16] = 4.0f;
        k4[j * 16] = (float)(j + 1);
        for (int c = 0; c < 16; ++c) v4[j * 16 + c] = 10.0f * (j + 1);
    }
    double o4[4 * 16];
    CHECK(kev_oracle_prefill(q4, k4, v4, 1, cu4, 1, 1, 1, 16, o4, 1) == 0);
    CHECK(fabs(o4[3 * 16] - 34.926527) < 5e-7);
    CHECK(o4[0] == 10.0);
}

static void decode_cases(void)
{
    /* bf16 slot decode: L = 1 (empty cache), L = capacity, a middle length; pool after */
    const int32_t NS = 4, CAP = 9, HK = 2, D = 8, H = 4, NR = 3;
    const size_t pool_n = (size_t)NS * 2 * HK * CAP * D;
    uint16_t *pool = bf16_buf(pool_n), *after = malloc(pool_n * sizeof(uint16_t));
    uint16_t *q = bf16_buf((size_t)NR * H * D), *kn = bf16_buf((size_t)NR * HK * D), *vn = bf16_buf((size_t)NR * HK * D);
    const int32_t ids[] = {2, 0, 3}, lens[] = {1, CAP, 5};
    double *out = malloc((size_t)NR * H * D * sizeof(double));
    CHECK(kev_oracle_decode(q, pool, NS, CAP, HK, D, ids, lens, kn, vn, NR, H, 0, out, after, 0) == 0);
    for (int h = 0; h < H; ++h)   /* L = 1: the new value row */
        for (int c = 0; c < D; ++c) {
            uint32_t u = (uint32_t)vn[((size_t)0 * HK + h / 2) * D + c] << 16;
            float f;
            memcpy(&f, &u, 4);
            CHECK(out[((size_t)0 * H + h) * D + c] == (double)f);
        }
    /* decode equals the last row of a prefill over the slot's rows */
    {
        const int32_t L = lens[2];
        uint16_t *kk = malloc((size_t)L * HK * D * 2), *vv = malloc((size_t)L * HK * D * 2);
        for (int p = 0; p < L; ++p)
            for (int g = 0; g < HK; ++g)
                for (int c = 0; c < D; ++c) {
                    kk[((size_t)p * HK + g) * D + c] = after[((((size_t)ids[2] * 2 + 0) * HK + g) * CAP + p) * D + c];
                    vv[((size_t)p * HK + g) * D + c] = after[((((size_t)ids[2] * 2 + 1) * HK + g) * CAP + p) * D + c];
                }
        uint16_t *qq = calloc((size_t)L * H * D, 2);
        memcpy(qq + (size_t)(L - 1) * H * D, q + (size_t)2 * H * D, (size_t)H * D * 2);
        const int32_t cu[] = {0, L};
        double *full = malloc((size_t)L * H * D * sizeof(double));
        CHECK(kev_oracle_prefill(qq, kk, vv, 0, cu, 1, H, HK, D, full, 1) == 0);
        for (int i = 0; i < H * D; ++i) CHECK(fabs(full[(size_t)(L - 1) * H * D + i] - out[(size_t)2 * H * D + i]) < 1e-12);
        free(kk), free(vv), free(qq), free(full);
    }
    const int32_t over[] = {1, CAP + 1, 5}, dup[] = {2, 2, 3};
    CHECK(kev_oracle_decode(q, pool, NS, CAP, HK, D, ids, over, kn, vn, NR, H, 0, out, after, 0) == -4);
    CHECK(kev_oracle_decode(q, pool, NS, CAP, HK, D, dup, lens, kn, vn, NR, H, 0, out, after, 0) == -5);

    /* paged decode through blocks of one row, scattered */
    const int32_t B = 1, NB = 20, MAXB = CAP;
    const size_t ppool_n = (size_t)NB * 2 * HK * B * D;
    uint16_t *ppool = bf16_buf(ppool_n), *pafter = malloc(ppool_n * 2);
    int32_t *tables = malloc((size_t)NR * MAXB * sizeof(int32_t));
    int32_t next = 0;
    const int32_t plens[] = {1, 3, 9};
    for (int r = 0; r < NR; ++r)
        for (int j = 0; j < MAXB; ++j) tables[r * MAXB + j] = j < plens[r] ? (next++ * 7) % NB : -1;
    CHECK(kev_oracle_paged_decode(q, ppool, NB, B, HK, D, tables, MAXB, plens, kn, vn, NR, H, 0, out, pafter, 0) == 0);
    const int32_t plong[] = {1, 3, MAXB * B + 1};
    CHECK(kev_oracle_paged_decode(q, ppool, NB, B, HK, D, tables, MAXB, plong, kn, vn, NR, H, 0, out, pafter, 0) != 0);
    free(pool), free(after), free(q), free(kn), free(vn), free(out), free(ppool), free(pafter), free(tables);
}

static void slot_prefill_cases(void)
{
    /* store into slots, then a chunk with an empty prefix and one that fills its slot */
    const int32_t NS = 5, CAP = 12, HK = 2, D = 8, H = 4;
    const int32_t cu[] = {0, 3, 3, 12};
    const int32_t n_seg = 3, T = 12;
    const size_t pool_n = (size_t)NS * 2 * HK * CAP * D;
    uint16_t *pool = bf16_buf(pool_n), *after = malloc(pool_n * 2);
    uint16_t *q = bf16_buf((size_t)T * H * D), *k = bf16_buf((size_t)T * HK * D), *v = bf16_buf((size_t)T * HK * D);
    const int32_t ids[] = {4, 1, 0};
    CHECK(kev_oracle_store_kv(k, v, 0, cu, n_seg, HK, D, ids, pool, NS, CAP, after) == 0);
    const int32_t pre[] = {0, 12, 3};
    double *out = malloc((size_t)T * H * D * sizeof(double));
    CHECK(kev_oracle_chunked_prefill(q, k, v, 0, cu, n_seg, H, HK, D, ids, pre, pool, NS, CAP, out, after, 0) == 0);
    const int32_t pre_over[] = {0, 0, 4};
    CHECK(kev_oracle_chunked_prefill(q, k, v, 0, cu, n_seg, H, HK, D, ids, pre_over, pool, NS, CAP, out, after, 0) == -4);
    const int32_t bad_ids[] = {4, 5, 0};
    CHECK(kev_oracle_store_kv(k, v, 0, cu, n_seg, HK, D, bad_ids, pool, NS, CAP, after) == -5);
    free(pool), free(after), free(q), free(k), free(v), free(out);
}

int main(void)
{
    prefill_cases();
    decode_cases();
    slot_prefill_cases();
    if (failures) {
        fprintf(stderr, "%d oracle checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: all checks passed\n");
    return 0;
}
