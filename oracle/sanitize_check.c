/*
 * Memory and undefined-behaviour check of the CPU oracle (test
 * infrastructure): a small program that calls every oracle entry point on
 * seeded inputs with ragged lengths, partial and empty blocks, both element
 * types, invalid working-set rows and loaded slot tables.  The test suite
 * builds it together with oracle.c under -fsanitize=address,undefined and
 * runs it; any sanitizer report, or a failed property below, fails the run.
 * The properties are cheap cross-checks that hold by definition (a Quest
 * bound is never below the exact block max; attention over the pool equals
 * attention over the source up to the rounding of their different
 * normalisation order).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct oracle_lru oracle_lru;
int oracle_score_blockmax(int, int, int, int, int, int, int, int, const void *, const void *, const int32_t *,
                          double, int, double *);
int oracle_quest_meta(int, int, int, int, int, int, const void *, const int32_t *, int, double *);
int oracle_score_quest(int, int, int, int, int, int, int, const void *, const void *, int, const int32_t *, int,
                       double, int, double *);
int oracle_topk(int, int, int, const double *, const int32_t *, int, int, int, int, int, int32_t *, int32_t *);
oracle_lru *oracle_lru_create(int, int);
void oracle_lru_destroy(oracle_lru *);
void oracle_lru_flush(oracle_lru *);
void oracle_lru_get(const oracle_lru *, int32_t *);
void oracle_lru_order(const oracle_lru *, int32_t *);
void oracle_lru_load(oracle_lru *, const int32_t *, const uint32_t *);
int oracle_lru_step(oracle_lru *, int, int, const int32_t *, const int32_t *, int32_t *, uint8_t *, int32_t *,
                    int32_t *, int32_t *);
int oracle_capped_step(int, int, int, int, int, const int32_t *, const int32_t *, const double *, int32_t *,
                       int32_t *, uint8_t *, int32_t *, int32_t *, int32_t *);
int oracle_check_state(int, int, int, const int32_t *, const uint32_t *, const uint32_t *, int32_t *);
int oracle_append(int, int, int, int, int, int, const void *, const void *, int32_t *, void *, void *,
                  const int32_t *, int, void *, void *);
int oracle_gather(int, int, int, int, int, int, int, const int32_t *, const int32_t *, const int32_t *, const void *,
                  const void *, void *, void *);
int oracle_attention(int, int, int, int, int, int, int, const void *, const void *, const void *, const int32_t *,
                     const int32_t *, int, const int32_t *, double, double *, double *);
int oracle_attention_pool(int, int, int, int, int, int, int, const void *, const void *, const void *,
                          const int32_t *, const int32_t *, const int32_t *, int, const int32_t *, double, double *,
                          double *);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) /* uniform in [-1, 1) */
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng_state >> 11) / (double)(1ull << 53) * 2.0 - 1.0;
}
static uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

static int failures = 0;
#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                  \
        }                                                                \
    } while (0)

static void run(int dtype)
{
    const int B = 3, Hq = 8, Hkv = 2, D = 16, T = 80, blk = 16, NB = T / blk, NQ = 2, k = 3, C = 4;
    const int P = B * Hkv, eb = dtype ? 2 : 4;
    const int32_t lens[3] = {80, 37, 0}; /* full, partial last block, empty */
    const size_t nkv = (size_t)B * Hkv * T * D, nq = (size_t)B * NQ * Hq * D;
    void *K = malloc(nkv * eb), *V = malloc(nkv * eb), *q = malloc(nq * eb), *qa = malloc((size_t)B * Hq * D * eb);
    for (size_t i = 0; i < nkv; ++i) {
        float a = (float)urand(), b = (float)urand();
        if (dtype) {
            ((uint16_t *)K)[i] = to_bf16(a);
            ((uint16_t *)V)[i] = to_bf16(b);
        } else {
            ((float *)K)[i] = a;
            ((float *)V)[i] = b;
        }
    }
    for (size_t i = 0; i < nq; ++i) {
        float a = (float)urand();
        if (dtype)
            ((uint16_t *)q)[i] = to_bf16(a);
        else
            ((float *)q)[i] = a;
    }
    memcpy(qa, q, (size_t)B * Hq * D * eb); /* attention queries [B, Hq, D]: any seeded values */

    double *sc = malloc(sizeof(double) * P * NB), *sq = malloc(sizeof(double) * P * NB);
    double *meta = malloc(sizeof(double) * P * NB * 2 * D);
    CHECK(oracle_score_blockmax(B, NQ, Hq, Hkv, D, T, blk, dtype, q, K, lens, 0.25, NB, sc) == 0);
    CHECK(oracle_quest_meta(B, Hkv, D, T, blk, dtype, K, lens, NB, meta) == 0);
    CHECK(oracle_score_quest(B, NQ, Hq, Hkv, D, blk, dtype, q, meta, 2, lens, T, 0.25, NB, sq) == 0);
    for (int i = 0; i < P * NB; ++i)
        CHECK(isinf(sc[i]) ? isinf(sq[i]) : sq[i] >= sc[i] - 1e-12);
    /* one-token blocks of the empty sequence score -inf */
    {
        double s1[6 * 80];
        CHECK(oracle_score_blockmax(B, 1, Hq, Hkv, D, T, 1, dtype, q, K, lens, 1.0, T, s1) == 0);
        CHECK(isinf(s1[2 * Hkv * T]) && !isinf(s1[0]));
    }

    int32_t sel[6 * 3], cnt[6];
    CHECK(oracle_topk(B, Hkv, NB, sc, lens, T, blk, k, 0, 0, sel, cnt) == 0);
    CHECK(cnt[4] == 0 && cnt[2] == 3);
    CHECK(oracle_topk(B, Hkv, NB, sc, lens, T, blk, k, 4, 16, sel, cnt) == 0);
    CHECK(oracle_topk(B, Hkv, NB, sc, lens, T, blk, 1, 4, 16, sel, cnt) != 0); /* forced exceed the budget */
    CHECK(oracle_topk(B, Hkv, NB, sc, lens, T, blk, k, 0, 0, sel, cnt) == 0);

    int32_t ss[6 * 3], mb[6 * 3], ms[6 * 3], mc[6], table[6 * 4], order[6 * 4];
    uint8_t sh[6 * 3];
    oracle_lru *h = oracle_lru_create(P, C);
    for (int step = 0; step < 3; ++step)
        CHECK(oracle_lru_step(h, k, NB, sel, cnt, ss, sh, mb, ms, mc) == 0);
    oracle_lru_get(h, table);
    oracle_lru_order(h, order);
    uint32_t stamps[6 * 4];
    for (int i = 0; i < P * C; ++i)
        stamps[i] = (uint32_t)(i % 3);
    table[1] = table[0] >= 0 ? table[0] : 2; /* row 0: a block held twice */
    table[0] = table[1];
    table[C + 0] = NB;                        /* row 1: an id past the end */
    {
        uint32_t clk[6] = {2, 2, 2, 2, 2, 2};
        int32_t fl[6];
        CHECK(oracle_check_state(P, C, NB, table, stamps, clk, fl) >= 2 && (fl[0] & 2) && (fl[1] & 1));
    }
    oracle_lru_load(h, table, stamps);
    CHECK(oracle_lru_step(h, k, NB, sel, cnt, ss, sh, mb, ms, mc) == 0);
    CHECK(mc[0] == -1 && mc[1] == -1 && ss[0] == -1 && mb[0] == -1);
    int32_t bad_sel[6 * 3];
    memcpy(bad_sel, sel, sizeof bad_sel);
    bad_sel[2 * 3 + 1] = bad_sel[2 * 3]; /* row 2: not ascending */
    CHECK(oracle_lru_step(h, k, NB, bad_sel, cnt, ss, sh, mb, ms, mc) == 0 && mc[2] == -1);
    oracle_lru_flush(h);
    CHECK(oracle_lru_step(h, k, NB, sel, cnt, ss, sh, mb, ms, mc) == 0 && mc[2] == cnt[2]);

    int32_t capped[6 * 4];
    for (int i = 0; i < P * C; ++i)
        capped[i] = -1;
    for (int step = 0; step < 2; ++step)
        CHECK(oracle_capped_step(P, C, k, NB, NB, sel, cnt, sc, capped, ss, sh, mb, ms, mc) == 0);
    capped[C + 1] = capped[C + 0] >= 0 ? capped[C + 0] : 1;
    capped[C + 0] = capped[C + 1];
    CHECK(oracle_capped_step(P, C, k, NB, NB, sel, cnt, sc, capped, ss, sh, mb, ms, mc) == 0 && mc[1] == -1);

    void *pk = calloc((size_t)P * C * blk * D, eb), *pv = calloc((size_t)P * C * blk * D, eb);
    oracle_lru_flush(h);
    CHECK(oracle_lru_step(h, k, NB, sel, cnt, ss, sh, mb, ms, mc) == 0);
    CHECK(oracle_gather(P, C, T, D, eb, blk, k, mb, ms, mc, K, V, pk, pv) == 0);
    double *o1 = malloc(sizeof(double) * B * Hq * D), *o2 = malloc(sizeof(double) * B * Hq * D);
    double l1[3 * 8], l2[3 * 8];
    CHECK(oracle_attention(B, Hq, Hkv, D, T, blk, dtype, qa, K, V, sel, cnt, k, lens, 0.25, o1, l1) == 0);
    CHECK(oracle_attention_pool(B, Hq, Hkv, D, C, blk, dtype, qa, pk, pv, sel, ss, cnt, k, lens, 0.25, o2, l2) == 0);
    for (int i = 0; i < B * Hq * D; ++i)
        CHECK(fabs(o1[i] - o2[i]) <= 1e-12);
    for (int i = 0; i < B * Hq; ++i)
        CHECK((isinf(l1[i]) && isinf(l2[i])) || fabs(l1[i] - l2[i]) <= 1e-12);

    int32_t grow[3] = {79, 37, 0};
    void *nk = malloc((size_t)B * Hkv * D * eb), *nv = malloc((size_t)B * Hkv * D * eb);
    memset(nk, 0x3c, (size_t)B * Hkv * D * eb);
    memset(nv, 0x41, (size_t)B * Hkv * D * eb);
    oracle_lru_get(h, table);
    for (int rep = 0; rep < 3; ++rep) /* the first sequence fills its last token, then stays full */
        CHECK(oracle_append(B, Hkv, D, T, blk, eb, nk, nv, grow, K, V, table, C, pk, pv) == 0);
    CHECK(grow[0] == 80 && grow[1] == 40 && grow[2] == 3);
    CHECK(oracle_append(B, Hkv, D, T, blk, eb, nk, nv, grow, K, V, NULL, 0, NULL, NULL) == 0);

    oracle_lru_destroy(h);
    free(K), free(V), free(q), free(qa), free(sc), free(sq), free(meta), free(pk), free(pv), free(o1), free(o2);
    free(nk), free(nv);
}

int main(void)
{
    run(0);
    run(1);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run ok\n");
    return 0;
}
