// CPU check of the index arithmetic the kernels share with the host code
// (sampler_internal.h), over every legal tile length and a spread of vocab
// sizes up to the library's maximum.  Built with AddressSanitizer and UBSan
// by the test suite; any failed check prints its case and exits non-zero.
//
// What is checked, and where the kernels rely on it:
//   plan     every wave sub-slot of a row fits the row's candidate area
//            (4 nt wcap <= ROWCAP, wcap >= 1): the pass writes candidate e
//            of sub-slot s at s * wcap + e, e < wcap;
//   lds      the merge's dynamic LDS (rows_lds_words) never exceeds that of
//            the longest row at the shortest tile, the case the kernel file
//            bounds at compile time;
//   dense    every vocab id maps to a tile below ntd and a position below
//            DTILE, one id per (tile, position): the dense writer's bitmap
//            tb[DTILE / 32] and its rank words are indexed by that position;
//   est      the sample runs of the admission estimate lie inside the row,
//            start on a multiple of VEC, inside their own segment, and do
//            not overlap;
//   tiles    the full-row search's tiling of a short queue: with T > 1
//            tiles per row, the T tiles of TL elements (a multiple of the
//            passes' 4096-element step) cover the row, none empty; T stays
//            within FB_TILES_MAX; the tiles of all nq rows (slots qi T + t)
//            fit the grid, hence the partial slots the workspace holds, and
//            every queued row's arrival counter (index qi) is below FB_GRID;
//   exp      the table-driven exp the full-row search weighs elements
//            with (exp_neg_tab) against long-double exp: within 1.5 units in
//            the last place above the subnormal range, over 4 million
//            arguments in [-745, 0] (uniform, log-spaced towards 0, and
//            the ends of each table interval), exactly 1 at 0, and tiny
//            (below 2^-1000) from -745 down to -1000 and beyond;
//   prefix   the six-ballot bit-plane prefix of the staged select gives
//            every lane the exclusive prefix of the lanes' counts (at most
//            4 PASS_D = 32 each), so entries land in [cnt, cnt + total).
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <vector>

#include "sampler.h"
#include "sampler_internal.h"

using namespace smp;

static int failures = 0;

#define CHECK(cond, ...)                                          \
    do {                                                          \
        if (!(cond)) {                                            \
            if (failures < 20) {                                  \
                fprintf(stderr, "FAIL %s:%d: %s | ", __FILE__, __LINE__, #cond); \
                fprintf(stderr, __VA_ARGS__);                     \
                fprintf(stderr, "\n");                            \
            }                                                     \
            ++failures;                                           \
        }                                                         \
    } while (0)

// Vocab sizes: small ones densely, then the edges of every power of two,
// every tile and dense-group multiple near the common vocabularies, and the
// maximum.
static std::vector<int32_t> vocab_set() {
    std::vector<int32_t> v;
    for (int32_t x = 1; x <= 5000; ++x) v.push_back(x);
    for (int e = 12; e <= 21; ++e)
        for (int d = -9; d <= 9; ++d) v.push_back((1 << e) + d);
    const int32_t common[] = {6400, 32000, 32064, 50257, 65024, 100352, 128256, 151936,
                              152064, 256000, 262144, 1 << 21};
    for (int32_t c : common)
        for (int d = -3; d <= 3; ++d) v.push_back(c + d);
    for (int32_t m = 2048; m <= (1 << 21); m += 2048 * 37) {
        v.push_back(m - 1);
        v.push_back(m);
        v.push_back(m + 1);
    }
    std::vector<int32_t> out;
    for (int32_t x : v)
        if (x >= 1 && x <= SAMPLER_VOCAB_MAX) out.push_back(x);
    return out;
}

static void check_plans(const std::vector<int32_t> &vs) {
    const KPlan worst = make_plan(SAMPLER_VOCAB_MAX, SEG_MIN, 1);
    for (int32_t seg = SEG_MIN; seg <= SEG_MAX; seg += SEG_MIN)
        for (int32_t V : vs) {
            const KPlan l = make_plan(V, seg, 256);
            CHECK(l.nt >= 1 && (int64_t)l.nt * seg >= V && (int64_t)(l.nt - 1) * seg < V,
                  "V=%d seg=%d nt=%d", V, seg, l.nt);
            CHECK(l.wcap >= 1, "V=%d seg=%d wcap=%d", V, seg, l.wcap);
            CHECK(4 * l.wcap <= TCAP_MAX, "V=%d seg=%d wcap=%d", V, seg, l.wcap);
            CHECK((int64_t)4 * l.nt * l.wcap <= ROWCAP, "V=%d seg=%d nt=%d wcap=%d", V, seg,
                  l.nt, l.wcap);
            CHECK(l.ntd >= 1 && (int64_t)l.ntd * DTILE >= V, "V=%d ntd=%d", V, l.ntd);
            CHECK(rows_lds_words(l) <= rows_lds_words(worst), "V=%d seg=%d words=%d", V, seg,
                  rows_lds_words(l));
            CHECK(rows_lds_words(l) >= 4 * l.nt + 1 && rows_lds_words(l) >= l.ntd + 1,
                  "V=%d seg=%d", V, seg);
        }
}

// The automatic tile length: a multiple of SEG_MIN up to SEG_DEFAULT; below
// SEG_DEFAULT the grid stays within AUTO_WG_PER_CU workgroups per CU with at
// most AUTO_TILES_MAX tiles per row, it is the shortest such length, and the
// call's tile records fit the handle's workspace bound.
static int64_t auto_cases = 0;

static void check_auto_seg(const std::vector<int32_t> &vs) {
    const int32_t batches[] = {1, 2, 3, 4, 7, 16, 64, 100, 256, 1000, 1024, 4096};
    const int32_t cuss[] = {1, 80, 256, 304};
    for (int32_t cu : cuss)
        for (int32_t V : vs)
            for (int32_t B : batches) {
                const int32_t s = auto_seg(B, V, cu);
                CHECK(s >= SEG_MIN && s <= SEG_DEFAULT && s % SEG_MIN == 0, "B=%d V=%d seg=%d", B,
                      V, s);
                const KPlan l = make_plan(V, s, cu);
                if (s < SEG_DEFAULT) {
                    CHECK(l.nt <= AUTO_TILES_MAX && (int64_t)B * l.nt <= (int64_t)AUTO_WG_PER_CU * cu,
                          "B=%d V=%d seg=%d nt=%d", B, V, s, l.nt);
                    CHECK(l.wcap >= ROWCAP / (4 * AUTO_TILES_MAX), "B=%d V=%d wcap=%d", B, V, l.wcap);
                }
                for (int32_t t = SEG_MIN; t < s; t += SEG_MIN) {
                    const KPlan lt = make_plan(V, t, cu);
                    CHECK(lt.nt > AUTO_TILES_MAX || (int64_t)B * lt.nt > (int64_t)AUTO_WG_PER_CU * cu,
                          "B=%d V=%d: %d fits before %d", B, V, t, s);
                }
                // the handle's bound, for any max_batch >= B
                const KPlan ld = make_plan(V, SEG_DEFAULT, cu);
                const int64_t bound = std::max((int64_t)B * ld.nt, (int64_t)AUTO_WG_PER_CU * cu);
                CHECK((int64_t)B * l.nt <= bound, "B=%d V=%d records", B, V);
                ++auto_cases;
            }
}

// Every id of a row of V maps into its tile, inside DTILE, and no two ids
// share a (tile, position).
static int64_t dense_ids = 0;

static void check_dense(int32_t V) {
    const KPlan l = make_plan(V, SEG_DEFAULT, 256);
    const uint32_t ntd = (uint32_t)l.ntd;
    std::vector<uint8_t> seen((size_t)ntd * DTILE, 0);
    for (uint32_t j = 0; j < (uint32_t)V; ++j) {
        const uint32_t t = dense_tile(j, ntd), pos = dense_pos(j, ntd);
        if (t >= ntd || pos >= (uint32_t)DTILE) {
            CHECK(false, "V=%d j=%u tile=%u pos=%u", V, j, t, pos);
            return;
        }
        uint8_t &s = seen[(size_t)t * DTILE + pos];
        CHECK(s == 0, "V=%d j=%u maps onto a used slot (tile %u pos %u)", V, j, t, pos);
        s = 1;
        // the bitmap word and bit of the position stay inside the tile's words
        CHECK((pos >> 5) < (uint32_t)(DTILE / 32), "V=%d j=%u", V, j);
        // the writer of tile t stores position pos of its LDS copy at element
        // (t + (pos / DGR) ntd) DGR + pos % DGR of the row: j itself
        const uint32_t back = (t + (pos / DGR) * ntd) * DGR + pos % DGR;
        CHECK(back == j, "V=%d j=%u written at %u", V, j, back);
    }
    dense_ids += V;
}

static void check_estimate(int32_t V) {
    if (V <= EST_N) return;
    for (int b = 0; b < 16; ++b) {
        int prev_end = 0;
        for (int s = 0; s < EST_SEGS; ++s) {
            const int st = est_run_start(s, b, V);
            const int64_t seg0 = ((int64_t)s * V / EST_SEGS) & ~(int64_t)(VEC - 1);
            CHECK(st >= 0 && st + EST_SEG <= V, "V=%d b=%d s=%d start=%d", V, b, s, st);
            CHECK(st % VEC == 0, "V=%d b=%d s=%d start=%d", V, b, s, st);
            CHECK(st >= seg0, "V=%d b=%d s=%d start=%d seg0=%lld", V, b, s, st,
                  (long long)seg0);
            CHECK(st >= prev_end, "V=%d b=%d s=%d overlaps the previous run", V, b, s);
            prev_end = st + EST_SEG;
        }
        // the offset pattern repeats every 16 rows
        for (int s = 0; s < EST_SEGS; ++s)
            CHECK(est_run_start(s, b, V) == est_run_start(s, b + 16, V), "V=%d b=%d s=%d", V,
                  b, s);
    }
}

// A wave of 64 lanes, each with n_l <= 32 admitted entries: bit plane k of
// the counts is one ballot; a lane's rank in it (set lanes below it) shifted
// by k, summed over the six planes, is its exclusive prefix.
static int64_t tilings = 0;
static void check_tiling(int32_t V) {
    static const int batches[] = {1, 2, 3, 4, 7, 15, 16, 17, 31, 64, 100, 255, 256, 257, 1024, 4096};
    for (int B : batches) {
        const int G = fb_grid(B);
        CHECK(G >= 1 && G <= FB_GRID && (B * FB_TILES_MAX >= FB_GRID || G == B * FB_TILES_MAX),
              "B=%d grid %d", B, G);
        const int nqmax = B < 600 ? B : 600;
        for (int nq = 0; nq <= nqmax; ++nq) {
            const FbTiling f = fb_tiling((uint32_t)nq, (uint32_t)G, V);
            ++tilings;
            CHECK(f.T >= 1 && f.T <= FB_TILES_MAX, "V=%d B=%d nq=%d T=%d", V, B, nq, f.T);
            if (f.T == 1) {
                CHECK(f.TL == V, "V=%d nq=%d TL=%d", V, nq, f.TL);
                continue;
            }
            CHECK(f.TL % FB_GROUP == 0, "V=%d nq=%d TL=%d", V, nq, f.TL);
            CHECK((int64_t)(f.T - 1) * f.TL < V && (int64_t)f.T * f.TL >= V,
                  "V=%d nq=%d T=%d TL=%d: a tile is empty or the row is not covered", V, nq, f.T,
                  f.TL);
            CHECK((int64_t)nq * f.T <= G, "V=%d B=%d nq=%d T=%d: slots beyond the grid", V, B,
                  nq, f.T);
            CHECK(nq - 1 < FB_GRID, "V=%d nq=%d: arrival counter out of range", V, nq);
        }
    }
}

static double exp_worst_ulp = 0.0;
static void check_exp(std::mt19937 &rng) {
    static const double tab[64] = {SMP_EXP2_J64_VALUES};
    auto one = [&](double t) {
        const double got = exp_neg_tab(t, tab);
        const long double ref = expl((long double)t);
        if (ref >= (long double)DBL_MIN) {
            const double ulp = ldexp(1.0, ilogb((double)ref) - 52);
            const double err = (double)fabsl((long double)got - ref) / ulp;
            if (err > exp_worst_ulp) exp_worst_ulp = err;
            CHECK(err <= 1.5, "t=%.17g got=%.17g ref=%.17Lg err=%.3g ulp", t, got, ref, err);
        } else {
            CHECK(got >= 0.0 && got < 0x1p-1000, "t=%.17g got=%.17g", t, got);
        }
    };
    std::uniform_real_distribution<double> uni(-745.0, 0.0), lg(-30.0, 3.0);
    for (int i = 0; i < 2000000; ++i) one(uni(rng));
    for (int i = 0; i < 2000000; ++i) one(-pow(10.0, lg(rng)));
    for (int n = -47000; n <= 0; ++n) {  // table interval ends
        const double c = n * (M_LN2 / 64.0);
        one(nextafter(c + M_LN2 / 128.0, 0.0));
        one(c - M_LN2 / 128.0);
    }
    CHECK(exp_neg_tab(0.0, tab) == 1.0, "exp(0)");
    CHECK(exp_neg_tab(-0.0, tab) == 1.0, "exp(-0)");
    for (double t : {-745.2, -800.0, -1000.0, -1e6, -1e300}) one(t);
}

static void check_prefix(std::mt19937 &rng) {
    std::uniform_int_distribution<int> cnt(0, 32), pick(0, 5);
    for (int trial = 0; trial < 20000; ++trial) {
        uint32_t n[64];
        const int mode = pick(rng);
        for (int l = 0; l < 64; ++l)
            n[l] = mode == 0 ? 32u : mode == 1 ? (uint32_t)(l & 1) * 32u : (uint32_t)cnt(rng);
        uint32_t pre[64] = {}, tot = 0;
        for (int bit = 0; bit < 6; ++bit) {
            uint64_t bal = 0;
            for (int l = 0; l < 64; ++l) bal |= (uint64_t)((n[l] >> bit) & 1u) << l;
            for (int l = 0; l < 64; ++l)
                pre[l] += (uint32_t)__builtin_popcountll(bal & ((1ull << l) - 1ull)) << bit;
            tot += (uint32_t)__builtin_popcountll(bal) << bit;
        }
        uint32_t run = 0;
        for (int l = 0; l < 64; ++l) {
            CHECK(pre[l] == run, "trial %d lane %d pre=%u expected %u", trial, l, pre[l], run);
            run += n[l];
        }
        CHECK(tot == run, "trial %d total %u expected %u", trial, tot, run);
        CHECK(tot <= 64u * 32u, "trial %d", trial);
    }
}

int main() {
    const std::vector<int32_t> vs = vocab_set();
    check_plans(vs);
    check_auto_seg(vs);
    int ndense = 0;
    for (size_t i = 0; i < vs.size(); ++i) {
        const int32_t V = vs[i];
        check_dense(V);
        ++ndense;
        check_estimate(V);
        if (i % 7 == 0 || V < 70000) check_tiling(V);
    }
    std::mt19937 rng(12345);
    check_prefix(rng);
    check_exp(rng);
    if (failures) {
        fprintf(stderr, "%d failed checks\n", failures);
        return 1;
    }
    printf("index checks ok: %zu vocab sizes, %d dense maps (%lld ids), %d tile lengths, "
           "%lld automatic tile choices, %lld search tilings, table exp within %.2f ulp\n",
           vs.size(), ndense, (long long)dense_ids, SEG_MAX / SEG_MIN, (long long)auto_cases,
           (long long)tilings, exp_worst_ulp);
    return 0;
}
