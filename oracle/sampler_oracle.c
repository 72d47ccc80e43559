/*
 * Plain CPU oracle for the batched logits-sampling post-process.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code with the HIP library.
 *
 * It computes the plain definition of what the pages describe, slowly and
 * obviously:
 *   - every row is fully sorted (qsort), no segments, no guess, no radix;
 *   - softmax, cumulative sums and sampling ratios are done in double.
 * The rolling top-k (Ascend torch_npu "npu_top_k_top_p_sample" page, topK
 * section, rolling formula with segment length v = 8*1024), the top-k guess
 * for top-p and its 1e4 early-exit rule (same page, topP section) reach the
 * same kept sets faster; they are deliberately absent here.
 *
 * Steps for one row, in the order the library applies them:
 *   O1  x_j = fp32(logit)  (bf16 widens exactly)
 *   O2  repetition penalty once per distinct history id in [0, V):
 *         x > 0 ? x / rho : x * rho          (MiniMind ch.10 sec. 10.7,
 *                                             and the C++ post-processing
 *                                             blog, repetition_penalty)
 *   O3  temperature: x / T when T != 1       (MiniMind ch.10 sec. 10.4)
 *   O3b -0 is replaced by +0 (a reading: the sign of a zero logit carries
 *       no meaning for sampling; it makes the kept value well defined)
 *   O4  total order: larger x first, equal x -> smaller vocab id first
 *       (descending sorts of the Ascend page; tie rule is a reading)
 *   O5  top-k active iff row bit0 and 1 <= k <= min(V, 1024): C = first k
 *       of the order, else C = whole row      (Ascend page, topK, range
 *                                             rule and Card(top_k_value)=k)
 *   O5' with the TOPK_TIES call flag, C also takes every element equal to
 *       the k-th value: C = { j : x_j >= the k-th largest value }
 *                                             (MiniMind sec. 10.5: logits
 *                                             below the k-th value of topk
 *                                             are masked, so ties stay)
 *   O6  e_i = exp(x_Ci - x_C0), Z = sum e_i   (softmax over the survivors,
 *                                             Ascend page, topK/topP)
 *   O7  top-p active iff row bit1 and p < 1 (NaN -> inactive): keep the
 *       shortest prefix of C whose probability mass reaches p; element 0 is
 *       always kept                          (MiniMind sec. 10.6 shifted
 *                                             mask; blog top_p "minimal
 *                                             set"; Ascend fallback mask)
 *   O8  pi_i = e_i / sum_{i in K} e_i         (softmax of the filtered row)
 *   O9  sample (row bit2 and q given): r_i = pi_i / (q[K_i] + eps), the
 *       output is the vocab id of the largest r, lowest id on exact ties
 *       (Ascend page, Sample section: probs/(q+eps), argmax, gather through
 *       logits_idx; q paired with candidates by vocab id -- a reading).
 *       With eps = 0 and q = 0 the ratio of a finite logit is +inf (IEEE
 *       positive / 0; the probability of a finite logit is positive even
 *       where its double exponential underflows); -inf logits have ratio 0.
 *       Sampling off: the output is K_0, the greedy argmax (MiniMind 10.8).
 *   O9' sample by inverse CDF instead (row bit2 and uniforms u given; q is
 *       not used): the output is K_{n-1} for the least n >= 1 whose
 *       inclusive cumulative probability S_n = sum_{i<n} pi_i reaches u[b];
 *       u <= 0 or NaN gives n = 1, and when rounding leaves S_|K| below u
 *       the last element of K is taken.  (MiniMind sec. 10.8 draws the
 *       token from the filtered softmax with torch.multinomial; with the
 *       caller's uniform this is that draw made by inverse CDF in the
 *       order of O4 -- a reading of how the draw is made.)
 *   O10 dense filtered logits: x_j at K, -inf elsewhere  (Ascend page,
 *       logits_top_kp_select scatter; MiniMind -inf masking)
 *   O11 dense probabilities: fp32(pi) at K, 0 elsewhere.
 *
 * Per-row diagnostics returned beside the outputs:
 *   nkept   |K|
 *   margin  top-p decision margin min(S_n* - p, p - S_{n*-1}) (n* > 1),
 *           S_1 - p (n* = 1), +inf when top-p is off
 *   gap     (r1 - r2) / r1 over the two largest ratios, +inf when there is
 *           no sampling, a single candidate, or an infinite largest ratio
 *           (q + eps == 0 exactly); for inverse-CDF sampling the
 *           decision margin min(S_n - u, u - S_{n-1}) instead (+inf when
 *           n = 1 by u <= 0)
 *
 * Build:  gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math
 *         -o liboracle.so sampler_oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

#define ROW_TOPK 1u
#define ROW_TOPP 2u
#define ROW_SAMPLE 4u

#define NEED_LOGITS 1u
#define NEED_PROBS 2u
#define TOPK_TIES 4u

#define TOPK_CAP 1024

typedef struct {
    float x;
    int32_t id;
} item_t;

/* O4: larger value first; equal values (IEEE ==, so -0 == +0) -> smaller id. */
static int order_cmp(const void *pa, const void *pb)
{
    const item_t *a = (const item_t *)pa;
    const item_t *b = (const item_t *)pb;
    if (a->x > b->x) return -1;
    if (a->x < b->x) return 1;
    return (a->id < b->id) ? -1 : (a->id > b->id) ? 1 : 0;
}

static float widen(const void *logits, int32_t dtype, int64_t off)
{
    if (dtype == ORACLE_BF16) {
        uint16_t h = ((const uint16_t *)logits)[off];
        uint32_t bits = (uint32_t)h << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return f;
    }
    return ((const float *)logits)[off];
}

/* Transformed logits of one row: O1, O2, O3, O3b. */
static void row_transform(float *x, int32_t V, int32_t dtype, const void *logits,
                          int64_t row_off, float temperature, float rho,
                          const int32_t *ids, int64_t id_begin, int64_t id_end,
                          unsigned char *seen)
{
    for (int32_t j = 0; j < V; j++) x[j] = widen(logits, dtype, row_off + j);

    if (rho != 1.0f && ids != NULL) {
        memset(seen, 0, (size_t)V);
        for (int64_t t = id_begin; t < id_end; t++) {
            int32_t id = ids[t];
            if (id >= 0 && id < V) seen[id] = 1; /* out-of-range ids: ignored */
        }
        for (int32_t j = 0; j < V; j++) {
            if (!seen[j]) continue;
            x[j] = (x[j] > 0.0f) ? x[j] / rho : x[j] * rho;
        }
    }
    if (temperature != 1.0f) {
        for (int32_t j = 0; j < V; j++) x[j] = x[j] / temperature;
    }
    for (int32_t j = 0; j < V; j++) {
        if (x[j] == 0.0f) x[j] = 0.0f; /* -0 -> +0 */
    }
}

/*
 * Process rows [row_begin, row_end).  Pointers are host pointers with the
 * layouts of the library's sampler_args: logits [B, ld] (fp32 or bf16 bits),
 * top_k [B], top_p [B], q [B, V], u [B] (NULL = sampling by the exponential
 * race with q), ids/offsets CSR history, row_flags [B]
 * (NULL = all stages on), out_idx [B], out_logits / out_probs [B, V] (may be
 * NULL), nkept / margin / gap [B] (may be NULL).
 * Returns 0, or -1 on an allocation failure or a bad argument.
 */
int oracle_run(int32_t B, int32_t V, int32_t dtype, const void *logits, int64_t ld,
               const int32_t *top_k, const float *top_p, const float *q, const float *u,
               float eps,
               float temperature, float rho, const int32_t *ids,
               const int64_t *offsets, const uint8_t *row_flags, uint32_t flags,
               int64_t *out_idx, float *out_logits, float *out_probs,
               int32_t *nkept, double *margin, double *gap,
               int32_t row_begin, int32_t row_end)
{
    if (B < 0 || V < 1 || ld < V || logits == NULL || out_idx == NULL) return -1;
    if (row_begin < 0 || row_end > B || row_begin > row_end) return -1;

    float *x = (float *)malloc(sizeof(float) * (size_t)V);
    item_t *ord = (item_t *)malloc(sizeof(item_t) * (size_t)V);
    double *e = (double *)malloc(sizeof(double) * (size_t)V);
    unsigned char *seen = (unsigned char *)malloc((size_t)V);
    if (!x || !ord || !e || !seen) {
        free(x); free(ord); free(e); free(seen);
        return -1;
    }

    for (int32_t b = row_begin; b < row_end; b++) {
        uint32_t rf = row_flags ? row_flags[b] : (ROW_TOPK | ROW_TOPP | ROW_SAMPLE);
        int64_t id_begin = 0, id_end = 0;
        if (ids != NULL && offsets != NULL) {
            id_begin = offsets[b];
            id_end = offsets[b + 1];
        }
        row_transform(x, V, dtype, logits, (int64_t)b * ld, temperature, rho,
                      ids, id_begin, id_end, seen);

        /* O4: full sort of the row. */
        for (int32_t j = 0; j < V; j++) {
            ord[j].x = x[j];
            ord[j].id = j;
        }
        qsort(ord, (size_t)V, sizeof(item_t), order_cmp);

        /* O5: candidate set C = ord[0 .. nC). */
        int32_t nC = V;
        if ((rf & ROW_TOPK) && top_k != NULL) {
            int32_t k = top_k[b];
            int32_t kmax = V < TOPK_CAP ? V : TOPK_CAP;
            if (k >= 1 && k <= kmax) {
                nC = k;
                if (flags & TOPK_TIES)
                    while (nC < V && ord[nC].x == ord[k - 1].x) nC++;
            }
        }

        /* O6: softmax over C in double. */
        double m = (double)ord[0].x;
        double Z = 0.0;
        for (int32_t i = 0; i < nC; i++) {
            e[i] = exp((double)ord[i].x - m);
            Z += e[i];
        }

        /* O7: shortest prefix with mass >= p. */
        int32_t nK = nC;
        double mrg = INFINITY;
        if ((rf & ROW_TOPP) && top_p != NULL && top_p[b] < 1.0f) {
            double p = (double)top_p[b];
            double S = 0.0, S_prev = 0.0;
            nK = nC;
            for (int32_t n = 1; n <= nC; n++) {
                S_prev = S;
                S += e[n - 1] / Z;
                if (S >= p) {
                    nK = n;
                    break;
                }
            }
            mrg = S - p;
            if (nK > 1 && p - S_prev < mrg) mrg = p - S_prev;
        }

        /* O8: renormalise over K. */
        double ZK = 0.0;
        for (int32_t i = 0; i < nK; i++) ZK += e[i];

        /* O9: exponential-race sample, O9': inverse-CDF sample, or greedy K_0. */
        int64_t idx = ord[0].id;
        double g = INFINITY;
        if ((rf & ROW_SAMPLE) && u != NULL) {
            double uu = (double)u[b];
            int32_t n = 1;
            if (uu > 0.0) {
                double S = 0.0, S_prev = 0.0;
                n = nK;
                for (int32_t i = 1; i <= nK; i++) {
                    S_prev = S;
                    S += e[i - 1] / ZK;
                    if (S >= uu) {
                        n = i;
                        break;
                    }
                }
                g = S - uu;
                if (n > 1 && uu - S_prev < g) g = uu - S_prev;
                if (g < 0.0) g = 0.0; /* rounding left S_|K| below u */
            }
            idx = ord[n - 1].id;
        } else if ((rf & ROW_SAMPLE) && q != NULL) {
            double r1 = -1.0, r2 = -1.0;
            int32_t best = -1;
            for (int32_t i = 0; i < nK; i++) {
                double pi = e[i] / ZK;
                int32_t id = ord[i].id;
                double den = (double)q[(int64_t)b * V + id] + (double)eps;
                /* a -inf logit has probability 0 and is never drawn; every
                 * finite logit has a positive probability (however far its
                 * double exponential underflows), so a zero denominator
                 * gives it an infinite ratio, as positive / 0 does in IEEE */
                double r;
                if (!(ord[i].x > -INFINITY)) r = 0.0;
                else if (den == 0.0) r = INFINITY;
                else r = pi / den;
                if (r > r1 || (r == r1 && id < best)) {
                    if (best >= 0) r2 = r1;
                    r1 = r;
                    best = id;
                } else if (r > r2) {
                    r2 = r;
                }
            }
            idx = best;
            /* infinite ratios come only from exact zeros of q + eps, and
             * their ties go to the lowest id: that decision has no
             * rounding in it, so it is not a near tie */
            if (nK > 1 && r2 >= 0.0)
                g = (r1 == INFINITY) ? INFINITY : (r1 > 0.0) ? (r1 - r2) / r1 : 0.0;
        }
        out_idx[b] = idx;
        if (nkept) nkept[b] = nK;
        if (margin) margin[b] = mrg;
        if (gap) gap[b] = g;

        /* O10 / O11: dense outputs. */
        if ((flags & NEED_LOGITS) && out_logits != NULL) {
            float *row = out_logits + (int64_t)b * V;
            for (int32_t j = 0; j < V; j++) row[j] = -INFINITY;
            for (int32_t i = 0; i < nK; i++) row[ord[i].id] = ord[i].x;
        }
        if ((flags & NEED_PROBS) && out_probs != NULL) {
            float *row = out_probs + (int64_t)b * V;
            for (int32_t j = 0; j < V; j++) row[j] = 0.0f;
            for (int32_t i = 0; i < nK; i++) row[ord[i].id] = (float)(e[i] / ZK);
        }
    }

    free(x);
    free(ord);
    free(e);
    free(seen);
    return 0;
}
