// Internal interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace smp {

// Streaming pass: one workgroup per tile of `seg` elements of a row.
constexpr int SEG_DEFAULT = 8192;  // the segment length v of the pages' rolling top-k
constexpr int SEG_MIN = 1024;
constexpr int SEG_MAX = 32768;
constexpr int ROWCAP = 8192;       // candidate entries per row, over all its tiles
constexpr int TCAP_MAX = 2048;     // candidate entries per tile (its four waves)
constexpr int WCAP_MAX = TCAP_MAX / 4;  // candidate entries per wave
constexpr int KMAX = 1024;         // largest k / guess
constexpr int VEC = 8;             // elements per group of the row helpers
// Row admission estimate: EST_SEGS runs of EST_SEG logits.
constexpr int EST_SEGS = 16;
constexpr int EST_SEG = 512;
constexpr int EST_N = EST_SEGS * EST_SEG;
constexpr int K1_THREADS = 512;    // estimate workgroup
// Row kernels.
constexpr int K3_THREADS = 1024;
constexpr int K3_BINS = 2048;      // value-space histogram bins
constexpr int K3_COLLECT = 4096;   // bucket members sorted in LDS
constexpr int K3_SEG = 65536;      // penalty-bitmap segment
// Full-row search over several workgroups: the first histogram level of a
// queued row is split into up to FB_TILES_MAX tiles of whole 4096-element
// groups, when the queue is short enough for the grid of FB_GRID workgroups.
constexpr int FB_GRID = 256;
constexpr int FB_TILES_MAX = 16;
constexpr int FB_GROUP = K3_THREADS * 4;  // elements of one step of the row passes
// One tile's partial histogram: masses, race keys, counts of the K3_BINS
// bins and the tile's total mass (padded to 256 bytes), then the mass sums
// and largest race keys of FB_CHUNKS chunks of consecutive bins.
constexpr int FB_CHUNKS = 64;
// Words of a queued row's synchronisation record (fbsync).
constexpr int FB_SYNC_WORDS = 4;
constexpr uint32_t FB_NO_BUCKET = 0xffffffffu;  // published: the tiles collect nothing
// Polls (one load and a short sleep each, about 1 us) a tile spends waiting
// for the row's bucket, and the last tile for the others' collections,
// before it gives up; giving up only costs speed.
constexpr int FB_POLLS = 200;
constexpr size_t FB_PART_CHUNKS = ((size_t)K3_BINS * (8 + 8 + 4) + 8 + 255) / 256 * 256;
constexpr size_t FB_PART_BYTES = (FB_PART_CHUNKS + (size_t)FB_CHUNKS * 16 + 255) / 256 * 256;
// Dense writer: a tile is DGR_PER_TILE group-rows of DGR elements (8 per
// lane of its workgroup).
constexpr int DGR_PER_TILE = 2;
constexpr int DGR_LOG2 = 11;
constexpr int DGR = 1 << DGR_LOG2;

// Row kinds written by the merge kernel.
enum RowKind : int32_t {
    KIND_UNFILTERED = 0,  // K = whole row; dense logits already written
    KIND_LIST = 1,        // K listed in klist[b][0..nK)
    KIND_FALLBACK = 2,    // guess failed; full-row cutoff search pending
    KIND_THRESH = 3,      // K = { comp >= T } (after the full-row search)
};

struct ChunkStat {
    float m;       // max transformed logit of the chunk (-inf if none)
    float xmin;    // min finite transformed logit (+inf if none)
    double z;      // sum exp(x - m) over the chunk
    float rx;      // race winner: logit
    float rqe;     // race winner: q + eps
    uint32_t ridx; // race winner: vocab id (0xffffffff = none)
    uint32_t nstr; // select tiles: handed-over entries above the row estimate
};

struct RowInfo {
    int32_t kind;
    int32_t nK;
    uint64_t T;    // threshold composite key (KIND_THRESH); for KIND_FALLBACK a
                   // floor of the search (0: none; only composites >= T count)
    double ZK;     // sum exp(x - m) over K
    float m;       // row max (transformed)
    float xmin;    // row min finite
    uint32_t idx0; // id of the row maximum (first in order)
    uint32_t pad;
};

struct KParams {
    const void *logits;
    int64_t ld;
    const int32_t *top_k;
    const float *top_p;
    const float *q;
    const float *u;  // [B] uniforms of inverse-CDF sampling, or null (race with q)
    const int32_t *ids;
    const int64_t *offsets;
    const int32_t *plen;  // [B] history lengths within the slots, or null (whole slots)
    const uint8_t *row_flags;
    int64_t *out_idx;
    float *out_logits;
    float *out_probs;
    float eps;
    float temperature;
    float rho;
    uint32_t flags;
    int32_t b0;  // first row of the launch (rows b0 .. b0 + B - 1)
    int32_t B;   // rows of the launch
    int32_t V;
    int32_t guess;
    int32_t pen;  // penalty stage active for the call
};

struct KPlan {
    int32_t seg;   // elements per pass tile (a multiple of 1024)
    int32_t nt;    // tiles per row
    int32_t wcap;  // candidate entries per wave sub-slot (4 nt wcap <= ROWCAP)
    int32_t ntd;   // dense tiles per row: ceil(ceil(V / DGR) / DGR_PER_TILE)
    int32_t cus;   // compute units of the device
};

// Index arithmetic shared by the host code, the kernels and the CPU checks of
// its bounds (constexpr functions are callable on both sides).

// The tiling of a row of V elements at tile length seg.
constexpr KPlan make_plan(int32_t vocab, int32_t seg, int32_t cus) {
    KPlan l{};
    l.cus = cus;
    l.seg = seg;
    l.nt = (int32_t)(((int64_t)vocab + seg - 1) / seg);
    const int64_t tc = ROWCAP / l.nt;
    l.wcap = (int32_t)((tc < TCAP_MAX ? tc : TCAP_MAX) / 4);
    const int64_t ngr = ((int64_t)vocab + DGR - 1) / DGR;  // dense group-rows
    l.ntd = (int32_t)((ngr + DGR_PER_TILE - 1) / DGR_PER_TILE);
    return l;
}

// The tile length of a call whose handle leaves it automatic: the shortest
// multiple of SEG_MIN below SEG_DEFAULT whose grid of batch x tiles stays
// within AUTO_WG_PER_CU workgroups per compute unit with at most
// AUTO_TILES_MAX tiles per row; SEG_DEFAULT when none does.  Small batches
// then spread each row over more compute units (the pass of a row of 32000
// runs on 32 workgroups instead of 4).  With at most AUTO_TILES_MAX tiles, a
// wave's share of the row's candidate capacity stays at least
// ROWCAP / (4 AUTO_TILES_MAX) = 32 entries.  Below SEG_DEFAULT a call has at
// most AUTO_WG_PER_CU cus tile records, so a workspace laid out for
// max(max_batch x tiles at SEG_DEFAULT, AUTO_WG_PER_CU cus) records serves
// every batch up to max_batch.
constexpr int AUTO_WG_PER_CU = 4;
constexpr int AUTO_TILES_MAX = 64;
constexpr int32_t auto_seg(int32_t batch, int32_t vocab, int32_t cus) {
    for (int32_t s = SEG_MIN; s < SEG_DEFAULT; s += SEG_MIN) {
        const int64_t nt = ((int64_t)vocab + s - 1) / s;
        if (nt <= AUTO_TILES_MAX && (int64_t)batch * nt <= (int64_t)AUTO_WG_PER_CU * cus) return s;
    }
    return SEG_DEFAULT;
}

// Dense writer tiles: group-row g (DGR elements) of a row belongs to tile
// g mod ntd, at position (g / ntd) DGR inside it.
constexpr int DTILE = DGR * DGR_PER_TILE;
constexpr uint32_t dense_tile(uint32_t j, uint32_t ntd) { return (j >> DGR_LOG2) % ntd; }
constexpr uint32_t dense_pos(uint32_t j, uint32_t ntd) {
    return (((j >> DGR_LOG2) / ntd) << DGR_LOG2) | (j & (uint32_t)(DGR - 1));
}
// First element of sample run s (of EST_SEGS) of row b of a row of V >
// EST_N elements: inside the s-th of EST_SEGS equal segments, at one of 16
// offsets that depend on s and b, a multiple of VEC.
constexpr int est_run_start(int s, int b, int V) {
    const int64_t seg0 = ((int64_t)s * V / EST_SEGS) & ~(int64_t)(VEC - 1);
    const int64_t seg1 = ((int64_t)(s + 1) * V / EST_SEGS) & ~(int64_t)(VEC - 1);
    const int64_t room = seg1 - seg0 - EST_SEG;  // >= 0 when V > EST_N
    const int64_t step = (room / 16) & ~(int64_t)(VEC - 1);
    return (int)(seg0 + (int64_t)((s * 5 + b * 3) & 15) * step);
}

// exp(t) for finite t <= 0 in double, by the table-driven method of P. T. P.
// Tang (ACM Trans. Math. Softw. 15(2), 1989): with n = rint(64 t / ln 2) =
// 64 k + j (0 <= j < 64), t = n ln2 / 64 + r, |r| <= ln2 / 128, and
// exp(t) = 2^k 2^(j/64) exp(r), exp(r) - 1 by its Taylor polynomial of
// degree 5 (remainder below 4e-17).  ln2 / 64 is split into a 36-bit head, exact
// times any |n| < 2^17, and a tail.  The 64 values 2^(j/64) are rounded to
// nearest; t below -1000 (exp(t) = 0 in double) is clamped there.  Within a
// few units in the last place of exp for results above the subnormal range;
// the CPU checks measure it against long-double exp.  Host and device run
// the same IEEE operations (fma, rint, ldexp) and get the same result.
#define SMP_EXP2_J64_VALUES \
    0x1.0000000000000p+0, 0x1.02c9a3e778061p+0, 0x1.059b0d3158574p+0, 0x1.0874518759bc8p+0, \
    0x1.0b5586cf9890fp+0, 0x1.0e3ec32d3d1a2p+0, 0x1.11301d0125b51p+0, 0x1.1429aaea92de0p+0, \
    0x1.172b83c7d517bp+0, 0x1.1a35beb6fcb75p+0, 0x1.1d4873168b9aap+0, 0x1.2063b88628cd6p+0, \
    0x1.2387a6e756238p+0, 0x1.26b4565e27cddp+0, 0x1.29e9df51fdee1p+0, 0x1.2d285a6e4030bp+0, \
    0x1.306fe0a31b715p+0, 0x1.33c08b26416ffp+0, 0x1.371a7373aa9cbp+0, 0x1.3a7db34e59ff7p+0, \
    0x1.3dea64c123422p+0, 0x1.4160a21f72e2ap+0, 0x1.44e086061892dp+0, 0x1.486a2b5c13cd0p+0, \
    0x1.4bfdad5362a27p+0, 0x1.4f9b2769d2ca7p+0, 0x1.5342b569d4f82p+0, 0x1.56f4736b527dap+0, \
    0x1.5ab07dd485429p+0, 0x1.5e76f15ad2148p+0, 0x1.6247eb03a5585p+0, 0x1.6623882552225p+0, \
    0x1.6a09e667f3bcdp+0, 0x1.6dfb23c651a2fp+0, 0x1.71f75e8ec5f74p+0, 0x1.75feb564267c9p+0, \
    0x1.7a11473eb0187p+0, 0x1.7e2f336cf4e62p+0, 0x1.82589994cce13p+0, 0x1.868d99b4492edp+0, \
    0x1.8ace5422aa0dbp+0, 0x1.8f1ae99157736p+0, 0x1.93737b0cdc5e5p+0, 0x1.97d829fde4e50p+0, \
    0x1.9c49182a3f090p+0, 0x1.a0c667b5de565p+0, 0x1.a5503b23e255dp+0, 0x1.a9e6b5579fdbfp+0, \
    0x1.ae89f995ad3adp+0, 0x1.b33a2b84f15fbp+0, 0x1.b7f76f2fb5e47p+0, 0x1.bcc1e904bc1d2p+0, \
    0x1.c199bdd85529cp+0, 0x1.c67f12e57d14bp+0, 0x1.cb720dcef9069p+0, 0x1.d072d4a07897cp+0, \
    0x1.d5818dcfba487p+0, 0x1.da9e603db3285p+0, 0x1.dfc97337b9b5fp+0, 0x1.e502ee78b3ff6p+0, \
    0x1.ea4afa2a490dap+0, 0x1.efa1bee615a27p+0, 0x1.f50765b6e4540p+0, 0x1.fa7c1819e90d8p+0,
constexpr double EXP_INV_L = 0x1.71547652b82fep+6;  // 64 / ln 2
constexpr double EXP_L1 = 0x1.62e42fefa0000p-7;     // ln 2 / 64, head
constexpr double EXP_L2 = 0x1.cf79abc9e3b3ap-46;    // ln 2 / 64 - EXP_L1
__host__ __device__ inline double exp_neg_tab(double t, const double *tab) {
    t = t < -1000.0 ? -1000.0 : t;
    const double n = rint(t * EXP_INV_L);
    double r = fma(-n, EXP_L1, t);
    r = fma(-n, EXP_L2, r);
    // exp(r) - 1 = r + r^2 (1/2 + r/6 + r^2/24 + r^3/120), added to the table
    // value by one fma so that its rounding is the last
    double s = fma(r, 1.0 / 120.0, 1.0 / 24.0);
    s = fma(s, r, 1.0 / 6.0);
    s = fma(s, r, 0.5);
    const double q = fma(s, r * r, r);
    const int ni = (int)n;
    const double tj = tab[ni & 63];
    return ldexp(fma(tj, q, tj), ni >> 6);
}

// Tiles per queued row of the full-row search and their length: with nq rows
// queued and a grid of G workgroups, T = G / nq tiles per row (1 to
// FB_TILES_MAX, no more than the row has 4096-element groups), each of TL
// elements (a multiple of FB_GROUP) but the last; T = 1 keeps one workgroup
// per row.  nq * T <= G whenever T > 1, so each workgroup takes one tile.
struct FbTiling {
    int T, TL;
};
constexpr FbTiling fb_tiling(uint32_t nq, uint32_t G, int V) {
    FbTiling f{1, V};
    if (nq == 0 || V <= 0) return f;
    uint32_t t = G / nq;
    if (t > (uint32_t)FB_TILES_MAX) t = FB_TILES_MAX;
    const int groups = (V + FB_GROUP - 1) / FB_GROUP;
    if (t > (uint32_t)groups) t = (uint32_t)groups;
    if (t < 2) return f;
    const int gpt = (groups + (int)t - 1) / (int)t;  // groups per tile
    f.TL = gpt * FB_GROUP;
    f.T = (V + f.TL - 1) / f.TL;
    if (f.T < 2) f = FbTiling{1, V};
    return f;
}

// Dynamic LDS words of the row merge: per-sub-slot candidate offsets, then
// per-dense-tile counts of the kept list.
constexpr int rows_lds_words(const KPlan &l) {
    return (l.nt * 4 > l.ntd ? l.nt * 4 : l.ntd) + 1;
}

struct KWork {
    uint64_t *cand;   // [maxB][ROWCAP]; sub-slot s (tile t, wave w: 4t + w) at s * wcap
    uint32_t *wcnt;   // [maxB][nt][4] entries | strict count << 16 (all ones: overflow)
    ChunkStat *cstat; // [maxB][nt][4] per-wave statistics / winners
    RowInfo *info;    // [maxB]
    uint64_t *klist;  // [maxB][KMAX] kept list of rows with a list, grouped by tile
    uint32_t *ktoff;  // [maxB][ntd + 1] start of each dense tile's group in klist
    float *rowthr;    // [maxB] estimated admission value of the row
    float *rowref;    // [maxB] transformed sample maximum (reference for exponentials)
    float *rowlo;     // [maxB] transformed smallest value of the estimate sample
    uint32_t *fbcnt;  // [1] rows queued for the full-row top-p search
    uint32_t *fblist; // [maxB] those rows
    uint32_t *fbsync;   // [FB_GRID][4] per queued row i (zeroed by the pass): tiles arrived,
                        // published bucket + 1 (or FB_NO_BUCKET), tiles done collecting,
                        // members listed
    char *fbpart;       // [fallback grid][FB_PART_BYTES] partial histograms of the tiles
};

// Workgroups of the full-row search for B rows: FB_GRID, or fewer when B rows
// cannot use them all.
constexpr int fb_grid(int B) {
    return B <= 0 ? 1 : (int64_t)B * FB_TILES_MAX < FB_GRID ? B * FB_TILES_MAX : FB_GRID;
}

// Decode-step epilogue over all rows of a call (one workgroup).
struct EpiParams {
    int64_t *out_idx;
    uint8_t *finished;       // or null
    int64_t eos;
    int32_t *ids;            // history slots (written when append is set)
    const int64_t *offsets;
    int32_t *len;            // history lengths (read / written when append is set)
    int32_t *counts;         // [2] or null
    int32_t B;
    int32_t append;
};
constexpr int EPI_THREADS = 1024;

// Launchers (sampler_kernels.hip).  Return hipSuccess or the launch error.
hipError_t launch_plan(const KParams &p, const KPlan &l, const KWork &w, int dtype, bool aligned,
                       hipStream_t s);
hipError_t launch_pass(const KParams &p, const KPlan &l, const KWork &w, int dtype, bool aligned,
                       hipStream_t s);
hipError_t launch_rows(const KParams &p, const KPlan &l, const KWork &w, hipStream_t s);
hipError_t launch_fallback(const KParams &p, const KPlan &l, const KWork &w, int dtype,
                           bool aligned, hipStream_t s);
hipError_t launch_dense(const KParams &p, const KPlan &l, const KWork &w, int dtype,
                        bool aligned, hipStream_t s);
hipError_t launch_epilogue(const EpiParams &e, hipStream_t s);

// The device address of the library's static workspace on `device` (the
// current device), SAMPLER_STATIC_SCRATCH_BYTES bytes; looked up once per
// device.
hipError_t static_scratch(int device, void **ptr);

}  // namespace smp
