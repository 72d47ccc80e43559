/*
 * Memory and undefined-behaviour check of the CPU oracle (oracle/
 * sampler_oracle.c), built with AddressSanitizer and UBSan by the test suite.
 *
 * Runs oracle_run over seeded random rows of many shapes, with every stage
 * switched on and off, both storage types, histories with out-of-range and
 * repeated ids, inverse-CDF and race sampling (eps = 0, zeros in q), ld > V,
 * row ranges and the edge cases outside the contract (all -inf rows, NaN
 * logits: only memory safety is asked of them).  Inputs are exactly sized
 * heap blocks, so a read or write past a row is an AddressSanitizer error.
 * In-contract rows are also checked for what any correct result satisfies:
 * the output id lies in the row and in the kept set, |K| is within [1, V],
 * the dense logits keep at most |K| finite entries and the probabilities sum
 * to one.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_run(int32_t B, int32_t V, int32_t dtype, const void *logits, int64_t ld,
               const int32_t *top_k, const float *top_p, const float *q, const float *u,
               float eps, float temperature, float rho, const int32_t *ids,
               const int64_t *offsets, const uint8_t *row_flags, uint32_t flags,
               int64_t *out_idx, float *out_logits, float *out_probs, int32_t *nkept,
               double *margin, double *gap, int32_t row_begin, int32_t row_end);

static int failures = 0;
#define CHECK(cond, ...)                                                        \
    do {                                                                        \
        if (!(cond)) {                                                          \
            if (failures < 30) {                                                \
                fprintf(stderr, "FAIL %s:%d: %s | ", __FILE__, __LINE__, #cond); \
                fprintf(stderr, __VA_ARGS__);                                   \
                fprintf(stderr, "\n");                                          \
            }                                                                   \
            ++failures;                                                         \
        }                                                                       \
    } while (0)

/* splitmix64 */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static double unif(void) { return (double)(next_u64() >> 11) * 0x1.0p-53; }
static int below(int n) { return (int)(next_u64() % (uint64_t)n); }
static float normal(void) {
    double a = unif(), b = unif();
    if (a < 1e-300) a = 1e-300;
    return (float)(sqrt(-2.0 * log(a)) * cos(6.283185307179586 * b));
}

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* mode: 0 in contract, 1 all -inf rows, 2 NaN entries */
static void one_case(int B, int V, int ldpad, int dtype, int mode, int variant) {
    const int64_t ld = (int64_t)V + ldpad;
    const size_t ne = (size_t)B * (size_t)ld;
    float *lf = (float *)xmalloc(sizeof(float) * ne);
    uint16_t *lb = (uint16_t *)xmalloc(sizeof(uint16_t) * ne);
    const float scale = variant % 3 == 0 ? 1.0f : variant % 3 == 1 ? 20.0f : 1e-3f;
    for (size_t i = 0; i < ne; ++i) {
        float x = normal() * scale;
        if (variant % 5 == 4) x = (float)below(4); /* heavy ties */
        if (mode == 1) x = -INFINITY;
        if (mode == 2 && below(7) == 0) x = NAN;
        if (mode == 0 && variant % 7 == 3 && below(9) == 0) x = -INFINITY;
        lf[i] = x;
        lb[i] = to_bf16(x);
        if (dtype == 1) {
            uint32_t w = (uint32_t)lb[i] << 16;
            memcpy(&lf[i], &w, 4);
        }
    }
    int32_t *top_k = (int32_t *)xmalloc(sizeof(int32_t) * (size_t)B);
    float *top_p = (float *)xmalloc(sizeof(float) * (size_t)B);
    float *q = (float *)xmalloc(sizeof(float) * (size_t)B * (size_t)V);
    float *u = (float *)xmalloc(sizeof(float) * (size_t)B);
    uint8_t *rf = (uint8_t *)xmalloc((size_t)B);
    int64_t *off = (int64_t *)xmalloc(sizeof(int64_t) * (size_t)(B + 1));
    int64_t *out_idx = (int64_t *)xmalloc(sizeof(int64_t) * (size_t)B);
    float *out_logits = (float *)xmalloc(sizeof(float) * (size_t)B * (size_t)V);
    float *out_probs = (float *)xmalloc(sizeof(float) * (size_t)B * (size_t)V);
    int32_t *nk = (int32_t *)xmalloc(sizeof(int32_t) * (size_t)B);
    double *margin = (double *)xmalloc(sizeof(double) * (size_t)B);
    double *gap = (double *)xmalloc(sizeof(double) * (size_t)B);
    int nids = 0;
    off[0] = 0;
    for (int b = 0; b < B; ++b) {
        const int kk = below(5);
        top_k[b] = kk == 0 ? 0 : kk == 1 ? 1 + below(V) : kk == 2 ? V + below(3)
                 : kk == 3 ? 1024 + below(5) : 1 + below(64);
        const int pp = below(6);
        top_p[b] = pp == 0 ? 1.0f : pp == 1 ? NAN : pp == 2 ? 0.0f : pp == 3 ? 1.5f
                 : (float)unif();
        u[b] = below(8) == 0 ? 0.0f : below(8) == 0 ? 1.0f : (float)unif();
        rf[b] = (uint8_t)below(8);
        nids += below(6);
        off[b + 1] = nids;
    }
    int32_t *ids = (int32_t *)xmalloc(sizeof(int32_t) * (size_t)(nids ? nids : 1));
    for (int t = 0; t < nids; ++t)
        ids[t] = below(10) == 0 ? -1 - below(3) : below(10) == 0 ? V + below(3) : below(V);
    for (size_t i = 0; i < (size_t)B * (size_t)V; ++i) {
        const int z = variant % 4;
        q[i] = z == 0 ? (float)(-log(1.0 - unif())) : z == 1 ? (float)exp(-60.0 + 65.0 * unif())
             : (below(3) == 0 ? 0.0f : (float)unif());
    }
    const float eps = variant % 2 ? 0.0f : 1e-20f;
    const float temp = variant % 3 == 2 ? 0.7f : 1.0f;
    const float rho = variant % 4 == 1 ? 1.3f : 1.0f;
    const int use_u = variant % 6 == 5;
    const uint32_t flags = (variant % 8 == 6) ? 4u | 3u : 3u;
    const int r0 = variant % 5 == 1 && B > 1 ? 1 : 0;

    const int rc = oracle_run(B, V, dtype, dtype ? (const void *)lb : (const void *)lf, ld,
                              variant % 9 == 8 ? NULL : top_k, top_p, q, use_u ? u : NULL, eps,
                              temp, rho, variant % 10 == 9 ? NULL : ids,
                              variant % 10 == 9 ? NULL : off, variant % 11 == 10 ? NULL : rf,
                              flags, out_idx, out_logits, out_probs, nk, margin, gap, r0, B);
    CHECK(rc == 0, "B=%d V=%d rc=%d", B, V, rc);
    if (mode == 0 && rc == 0)
        for (int b = r0; b < B; ++b) {
            const float *ol = out_logits + (size_t)b * V, *op = out_probs + (size_t)b * V;
            int finite = 0;
            double s = 0.0;
            for (int j = 0; j < V; ++j) {
                finite += ol[j] != -INFINITY;
                s += op[j];
            }
            CHECK(out_idx[b] >= 0 && out_idx[b] < V, "B=%d V=%d b=%d idx=%lld", B, V, b,
                  (long long)out_idx[b]);
            CHECK(nk[b] >= 1 && nk[b] <= V, "b=%d nkept=%d", b, nk[b]);
            /* a kept -inf logit (a row with few finite values) keeps -inf */
            CHECK(finite <= nk[b], "b=%d finite %d > nkept %d", b, finite, nk[b]);
            if (finite > 0) {
                CHECK(fabs(s - 1.0) < 1e-4, "b=%d prob sum %.9g", b, s);
                if (out_idx[b] >= 0 && out_idx[b] < V)
                    CHECK(ol[out_idx[b]] != -INFINITY, "b=%d sampled a dropped id", b);
            }
            /* margins are distances to a decision boundary; the inverse-CDF
               one is below zero only when rounding leaves S_|K| under u */
            CHECK(margin[b] >= 0.0, "b=%d margin %.9g", b, margin[b]);
            CHECK(use_u ? gap[b] >= -1e-12 : gap[b] >= 0.0, "b=%d gap %.9g", b, gap[b]);
        }
    /* argument errors are refused, not read */
    CHECK(oracle_run(B, 0, dtype, lf, ld, NULL, NULL, NULL, NULL, eps, 1.0f, 1.0f, NULL, NULL,
                     NULL, 0, out_idx, NULL, NULL, NULL, NULL, NULL, 0, B) == -1, "V=0");
    CHECK(oracle_run(B, V, dtype, lf, V - 1, NULL, NULL, NULL, NULL, eps, 1.0f, 1.0f, NULL,
                     NULL, NULL, 0, out_idx, NULL, NULL, NULL, NULL, NULL, 0, B) == -1, "ld<V");
    CHECK(oracle_run(B, V, dtype, lf, ld, NULL, NULL, NULL, NULL, eps, 1.0f, 1.0f, NULL, NULL,
                     NULL, 0, out_idx, NULL, NULL, NULL, NULL, NULL, 0, B + 1) == -1,
          "rows past B");
    free(lf); free(lb); free(top_k); free(top_p); free(q); free(u); free(rf); free(off);
    free(out_idx); free(out_logits); free(out_probs); free(nk); free(margin); free(gap);
    free(ids);
}

int main(void) {
    static const int shapes[][2] = {{1, 1}, {1, 2}, {3, 5}, {2, 64}, {4, 1000}, {3, 1025},
                                    {2, 2049}, {5, 4097}, {2, 20000}, {1, 70001}};
    int cases = 0;
    for (unsigned s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (int dtype = 0; dtype < 2; ++dtype)
            for (int variant = 0; variant < 24; ++variant) {
                one_case(shapes[s][0], shapes[s][1], variant % 3 == 1 ? 3 : 0, dtype, 0,
                         variant);
                ++cases;
            }
    for (int mode = 1; mode <= 2; ++mode)
        for (int variant = 0; variant < 12; ++variant) {
            one_case(3, 300, 0, variant & 1, mode, variant);
            ++cases;
        }
    if (failures) {
        fprintf(stderr, "%d failed checks\n", failures);
        return 1;
    }
    printf("oracle checks ok: %d cases\n", cases);
    return 0;
}
