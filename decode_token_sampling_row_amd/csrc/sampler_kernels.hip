// HIP kernels of the batched logits sampler (gfx950, wave64).
//
// Pipeline of one call (all on the caller's stream):
//
//   k_plan      grid = B.  Rows with top-k / top-p: an admission value from a
//               sample of the row (16 staggered runs of 512 logits), below
//               which no element can be among the row's kk largest with high
//               probability; the sample maximum as the reference for sums of
//               exponentials.
//   k_pass      grid = B x tiles of seg (8192 by default, the segment length
//               of the rolling top-k of the Ascend npu_top_k_top_p_sample
//               page, topK section).  Each workgroup reads one tile of one
//               row once from HBM: widen bf16 -> fp32, repetition penalty
//               (LDS bitmap of the tile's history ids), temperature.  Then,
//               each wave on its own:
//                 - rows with top-k / top-p: admit what reaches the row's
//                   admission value into the wave's LDS buffer and hand it
//                   over to the wave's sub-slot of the row; rows without
//                   top-k also sum exp(y - ref) (the softmax of that page's
//                   topP section);
//                 - rows that only sample: the exponential race over the
//                   tile, q streamed alongside;
//                 - greedy rows: the argmax;
//                 - the dense output of rows without a filter.
//   k_rows      grid = B.  Per row: the completeness check of what the pass
//               handed over (no wave overflowed its sub-slot, and at least kk
//               entries lie above the admission value's transform -- every
//               element left out lies at or below it); exact top-kk of the
//               candidates by radix select, softmax in double, the shortest
//               prefix reaching p (top-k guess accepted with a margin), the
//               exponential race over the kept set (gather of q at the kept
//               ids) or the inverse-CDF draw, output id, the kept list
//               grouped by tile.  Rows that fail the check, whose guess does
//               not settle top-p, or that draw by inverse CDF over the whole
//               row are queued.
//   k_fallback  grid = min(B, 256) over the queue.  The full-row search: a
//               value-space histogram of exp masses (or of counts, for the
//               exact kk-th element of a top-k row), key-space refinement,
//               an exact sort of the boundary bucket in LDS (or a rank among
//               ties by vocab id); then the race or the draw over the kept
//               set.  This is the page's full-sort fallback reached without a
//               full sort.
//   k_dense     grid = B x tiles, only when probabilities are asked for.
//               Writes them with full-line stores, composing each tile in
//               LDS from the kept list.
//   k_epilogue  one workgroup, when asked for.  The decode-step epilogue of
//               the MiniMind generation loop (sec. 10.9): finished rows
//               output EOS, rows that output EOS become finished, the output
//               is appended to the row's history slot, and the unfinished
//               rows are counted.
//
// Order and keys: a transformed logit x and its vocab id j form the 64-bit
// composite  (orderkey(x) << 32) | ~j ; larger composite = earlier in the
// row's order (larger value, then smaller id).  All composites of a row are
// distinct, so every selection below is exact and deterministic.

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "sampler.h"

#include "sampler_internal.h"

namespace smp {
namespace {

constexpr uint32_t NONE = 0xffffffffu;
constexpr uint32_t NEED_PROBS = 2u;
constexpr uint32_t TOPK_TIES = 4u;  // top-k keeps the ties at the k-th value
// top-p decisions taken from a guess must clear the cutoff by this much
// (relative to the row's total mass); the row's total is accumulated from
// fp32 exponentials, good to about 1e-6.  Rows inside the margin take the
// exact full-row search.
constexpr double GUESS_MARGIN = 1e-5;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- keys

__device__ __forceinline__ uint32_t f2key(float x) {
    const uint32_t b = __float_as_uint(x);
    return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
    uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(b);
}
__device__ __forceinline__ uint64_t mkcomp(float x, uint32_t j) {
    return ((uint64_t)f2key(x) << 32) | (uint64_t)(~j);
}
__device__ __forceinline__ uint32_t cidx(uint64_t c) { return ~(uint32_t)c; }
__device__ __forceinline__ float cval(uint64_t c) { return key2f((uint32_t)(c >> 32)); }

// ---------------------------------------------------------------- row mode

struct Mode {
    bool tk, tp;
    bool sm;   // samples by the exponential race with q
    bool inv;  // samples by inverse CDF with the caller's uniform u
    int k;
    float p;
};

__device__ __forceinline__ Mode row_mode(const KParams &P, int b) {
    // the three loads are independent of one another (one round trip)
    const uint32_t rf = P.row_flags ? (uint32_t)P.row_flags[b] : 7u;
    const int k = P.top_k ? P.top_k[b] : 0;
    const float p = P.top_p ? P.top_p[b] : 1.0f;
    const int kmax = P.V < KMAX ? P.V : KMAX;
    Mode md;
    md.tk = (rf & 1u) && P.top_k && k >= 1 && k <= kmax;
    md.k = md.tk ? k : 0;
    md.tp = (rf & 2u) && P.top_p && p < 1.0f;  // NaN compares false: stage off
    md.p = md.tp ? p : 1.0f;
    md.sm = (rf & 4u) && P.q && !P.u;
    md.inv = (rf & 4u) && P.u;
    return md;
}

// Penalty, temperature, -0 -> +0 (adding +0 maps -0 to +0 and leaves every
// other value unchanged).  Division is IEEE correctly rounded.  XF = false
// compiles the call without penalty or temperature down to the +0.
template <bool XF>
__device__ __forceinline__ float xform(float x, uint32_t hit, const KParams &P) {
    if (XF) {
        if (hit) x = (x > 0.0f) ? x / P.rho : x * P.rho;
        if (P.temperature != 1.0f) x = x / P.temperature;
    }
    return x + 0.0f;
}

// Row index of workgroup i in a grid of n row-workgroups: consecutive
// workgroups go round-robin to the 8 XCDs; give each XCD a contiguous block
// of rows so row-dependent work (stage mixes often cycle with the row) is
// spread evenly over the XCDs.
__device__ __forceinline__ int xcd_row(int i, int n) {
    int x = i & 7, pos = i >> 3;
    int q = n >> 3, r = n & 7;
    return x * q + (x < r ? x : r) + pos;
}

// ---------------------------------------------------------------- loads

template <int DT>
__device__ __forceinline__ float ld1(const void *p, int64_t j) {
    if (DT == 1) {
        uint32_t h = ((const uint16_t *)p)[j];
        return __uint_as_float(h << 16);
    }
    return ((const float *)p)[j];
}

// x[0..8) = elements j..j+8 of the row (nv valid).  Vector path when the
// row is 16-byte aligned and the group is whole.
template <int DT, bool AL>
__device__ __forceinline__ void load8(const void *p, int64_t j, int nv, float (&x)[8]) {
    if (AL && nv == 8) {
        if (DT == 1) {
            u32x4 u = __builtin_nontemporal_load((const u32x4 *)((const uint16_t *)p + j));
            x[0] = __uint_as_float(u.x << 16);
            x[1] = __uint_as_float(u.x & 0xffff0000u);
            x[2] = __uint_as_float(u.y << 16);
            x[3] = __uint_as_float(u.y & 0xffff0000u);
            x[4] = __uint_as_float(u.z << 16);
            x[5] = __uint_as_float(u.z & 0xffff0000u);
            x[6] = __uint_as_float(u.w << 16);
            x[7] = __uint_as_float(u.w & 0xffff0000u);
        } else {
            const f32x4 *q = (const f32x4 *)((const float *)p + j);
            f32x4 a = __builtin_nontemporal_load(q);
            f32x4 c = __builtin_nontemporal_load(q + 1);
            x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
            x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (i < nv) ? ld1<DT>(p, j + i) : 0.0f;
    }
}

// ---------------------------------------------------------------- wave / WG primitives

__device__ __forceinline__ uint32_t shx(uint32_t v, int m) {
    return (uint32_t)__shfl_xor((int)v, m, 64);
}
__device__ __forceinline__ uint64_t shx64(uint64_t v, int m) {
    uint32_t lo = shx((uint32_t)v, m), hi = shx((uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}
// The same exchange with lane ^ m on the vector ALU where gfx950 has a
// pattern for it (DPP quad permutes, the half-row mirror, a rotation of each
// row of 16 by 8, and the row and half-wave swaps), which avoids the LDS
// crossbar round trip of a shuffle.  m must be a constant once the caller's
// loops are unrolled, and every lane of the wave must be active: each lane
// reads its partner's register.
__device__ __forceinline__ uint32_t xlane(uint32_t v, int m) {
    const int lane = threadIdx.x & 63;
    switch (m) {
        case 1:  // quad_perm [1, 0, 3, 2]
            return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false);
        case 2:  // quad_perm [2, 3, 0, 1]
            return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false);
        case 4: {  // lane ^ 7 (half-row mirror), then lane ^ 3 (quad_perm [3, 2, 1, 0])
            const int t = __builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false);
            return (uint32_t)__builtin_amdgcn_update_dpp(0, t, 0x1B, 0xf, 0xf, false);
        }
        case 8:  // each row of 16 rotated by 8
            return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false);
        case 16: {  // odd rows swapped with even rows
            const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
            return (lane & 16) ? r[0] : r[1];
        }
        case 32: {  // upper half-wave swapped with the lower
            const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
            return (lane & 32) ? r[0] : r[1];
        }
        default:
            return shx(v, m);
    }
}
__device__ __forceinline__ uint64_t xlane64(uint64_t v, int m) {
    const uint32_t lo = xlane((uint32_t)v, m), hi = xlane((uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ double xlaned(double v, int m) {
    return __longlong_as_double((long long)xlane64((uint64_t)__double_as_longlong(v), m));
}
__device__ __forceinline__ float shxf(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ double shxd(double v, int m) { return __shfl_xor(v, m, 64); }

// Inclusive scans over the wave on the VALU: within each row of 16 lanes by
// DPP row shifts of 1, 2, 4 and 8 (a lane shifted in from outside the row
// adds 0), then the last lane of row 0 is added into row 1 and row 3's
// predecessor, and lane 31 into rows 2 and 3 (row broadcasts).  The lane
// layout was checked on the GPU against a serial prefix sum.  Every lane of
// the wave must be active.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_in0(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_in0d(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint64_t lo = dpp_in0<CTRL, ROWS>((uint32_t)u), hi = dpp_in0<CTRL, ROWS>((uint32_t)(u >> 32));
    return __longlong_as_double((long long)((hi << 32) | lo));
}
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v, int lane) {
    (void)lane;
    v += dpp_in0<0x111, 0xf>(v);  // row_shr:1
    v += dpp_in0<0x112, 0xf>(v);  // row_shr:2
    v += dpp_in0<0x114, 0xf>(v);  // row_shr:4
    v += dpp_in0<0x118, 0xf>(v);  // row_shr:8
    v += dpp_in0<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_in0<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}
__device__ __forceinline__ double wave_incl_scan_f64(double v, int lane) {
    (void)lane;
    v += dpp_in0d<0x111, 0xf>(v);
    v += dpp_in0d<0x112, 0xf>(v);
    v += dpp_in0d<0x114, 0xf>(v);
    v += dpp_in0d<0x118, 0xf>(v);
    v += dpp_in0d<0x142, 0xa>(v);
    v += dpp_in0d<0x143, 0xc>(v);
    return v;
}

// Exclusive prefix over the workgroup (thread order); total via `total`.
// sc: >= 16 LDS words.  Ends with a barrier so sc can be reused at once.
template <int NT>
__device__ __forceinline__ uint32_t wg_excl_scan_u32(uint32_t v, uint32_t *sc, uint32_t &total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t inc = wave_incl_scan_u32(v, lane);
    if (lane == 63) sc[w] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        uint32_t s = sc[i];
        before += (i < w) ? s : 0u;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return before + inc - v;
}

template <int NT>
__device__ __forceinline__ double wg_excl_scan_f64(double v, double *sc, double &total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    double inc = wave_incl_scan_f64(v, lane);
    if (lane == 63) sc[w] = inc;
    __syncthreads();
    double before = 0.0, tot = 0.0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        double s = sc[i];
        if (i < w) before += s;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return before + (inc - v);
}

template <int NT>
__device__ __forceinline__ double wg_sum_f64(double v, double *sc) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += xlaned(v, m);
    if ((threadIdx.x & 63) == 0) sc[threadIdx.x >> 6] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) t += sc[i];
    __syncthreads();
    return t;
}

template <int NT>
__device__ __forceinline__ uint64_t wg_max_u64(uint64_t v, uint64_t *sc) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o = xlane64(v, m);
        v = o > v ? o : v;
    }
    if ((threadIdx.x & 63) == 0) sc[threadIdx.x >> 6] = v;
    __syncthreads();
    uint64_t t = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) t = sc[i] > t ? sc[i] : t;
    __syncthreads();
    return t;
}

template <int NT>
__device__ __forceinline__ uint64_t wg_min_u64(uint64_t v, uint64_t *sc) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o = xlane64(v, m);
        v = o < v ? o : v;
    }
    if ((threadIdx.x & 63) == 0) sc[threadIdx.x >> 6] = v;
    __syncthreads();
    uint64_t t = ~0ull;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) t = sc[i] < t ? sc[i] : t;
    __syncthreads();
    return t;
}

template <int NT>
__device__ __forceinline__ uint32_t wg_min_u32(uint32_t v, uint32_t *sc) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = min(v, xlane(v, m));
    if ((threadIdx.x & 63) == 0) sc[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t t = NONE;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) t = min(t, sc[i]);
    __syncthreads();
    return t;
}

// Exponential race: is candidate a (logit xa, q+eps qa) ahead of b?
// e_a / qa > e_b / qb  <=>  (xa - xb) log2(e) > log2(qa) - log2(qb).  Equal
// ratios -> smaller id.  A zero q + eps gives a finite logit an infinite
// ratio (positive / 0); -inf logits never enter a race.
struct Race {
    float x, qe;
    uint32_t idx;
    float lq;  // log2(qe) when qe is a normal number in [2^-120, 2^120], else NaN
};

constexpr float LOG2E_F = 1.4426950408889634f;
// The fp32 decision quantity D = (xa - xb) log2 e - (log2 qa - log2 qb) is
// trusted when |D| exceeds this: with |xa - xb| <= 256 and |log2 q| <= 120
// its rounding error stays below 2^-10 (hardware log2 is good to a few ulp,
// the subtraction and the product to half an ulp each).  Closer calls are
// decided in double.
constexpr float RACE_BAND = 0.00390625f;  // 2^-8
constexpr float RACE_DMAX = 256.0f;

__device__ __forceinline__ float race_lq(float qe) {
    return (qe >= 7.52316385e-37f && qe <= 1.32922800e36f) ? __builtin_amdgcn_logf(qe)
                                                          : __builtin_nanf("");
}

// ln 2 as hi + lo, hi with 15 significant bits: k * hi is exact for |k| < 512
// (every exponent difference of two floats).
constexpr float LN2_HI = 0x1.62e4p-1f;
constexpr float LN2_LO = 0x1.7f7d1cp-20f;

// The close call, to about 1e-7 absolute in L = (xa - xb) - ln(qa / qb):
// zero denominators first (an infinite ratio; two of them tie), then xa - xb
// exactly as a two-term sum, ln(qa / qb) as the exponent difference times
// ln 2 (exact products) plus the log of the mantissa ratio, which lies in
// (0.5, 2) so that its absolute error stays at a few 1e-8.  Equal -> the
// smaller id.  Out of line: the fast test settles nearly every comparison,
// and the close call, inlined at each of the pass's offers, made up a sixth
// of the library's code (code that a call fetches again after its caches
// are flushed).
__device__ __attribute__((noinline)) bool race_ahead_exact(float xa, float qa, uint32_t ia, float xb, float qb,
                                                 uint32_t ib) {
    const bool za = qa == 0.0f, zb = qb == 0.0f;
    if (za || zb) return (za && zb) ? ia < ib : za;
    const float nb = -xb;
    const float dh = xa + nb;
    const float bb = dh - xa;
    const float dl = (xa - (dh - bb)) + (nb - bb);
    int ea, eb;
    const float ma = frexpf(qa, &ea), mb = frexpf(qb, &eb);
    const float k = (float)(ea - eb);
    const float A = dh - k * LN2_HI;
    const float B = dl - k * LN2_LO;
    const float L = (A - logf(ma / mb)) + B;
    return L > 0.0f || (L == 0.0f && ia < ib);
}

__device__ __forceinline__ bool race_ahead(const Race &a, const Race &b) {
    if (a.idx == NONE) return false;
    if (b.idx == NONE) return true;
    const float d = a.x - b.x;
    const float D = d * LOG2E_F - (race_lq(a.qe) - race_lq(b.qe));
    if (fabsf(d) <= RACE_DMAX) {
        if (D > RACE_BAND) return true;
        if (D < -RACE_BAND) return false;
    }
    return race_ahead_exact(a.x, a.qe, a.idx, b.x, b.qe, b.idx);
}

// Offer element (x, q + eps, id j) to a lane's running winner.  The usual
// candidate loses by far more than the band and costs a log2, a multiply
// and two compares.
__device__ __forceinline__ void race_offer(Race &best, float x, float qe, uint32_t j) {
    if (!(x > -INFINITY)) return;  // probability 0: never drawn
    const float lq = race_lq(qe);
    if (best.idx != NONE) {
        const float d = x - best.x;
        const float D = d * LOG2E_F - (lq - best.lq);
        const bool fast = fabsf(d) <= RACE_DMAX;
        if (fast && D < -RACE_BAND) return;
        if (!(fast && D > RACE_BAND) && !race_ahead_exact(x, qe, j, best.x, best.qe, best.idx))
            return;
    }
    best.x = x;
    best.qe = qe;
    best.idx = j;
    best.lq = lq;
}
// A candidate's race ratio in double, e = exp(x - max) over q + eps: 0 for a
// -inf logit (never drawn), +inf for a finite logit over a zero denominator.
__device__ __forceinline__ double race_ratio(float x, double e, double den) {
    if (!(x > -INFINITY)) return 0.0;
    return den == 0.0 ? (double)INFINITY : e / den;
}

template <int NT>
__device__ __forceinline__ Race wg_race(Race r, float *scx, float *scq, uint32_t *sci) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        Race o;
        o.x = shxf(r.x, m);
        o.qe = shxf(r.qe, m);
        o.idx = shx(r.idx, m);
        o.lq = 0.0f;
        if (race_ahead(o, r)) r = o;
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        scx[w] = r.x;
        scq[w] = r.qe;
        sci[w] = r.idx;
    }
    __syncthreads();
    Race t;
    t.x = scx[0];
    t.qe = scq[0];
    t.idx = sci[0];
    t.lq = 0.0f;
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) {
        Race o;
        o.x = scx[i];
        o.qe = scq[i];
        o.idx = sci[i];
        o.lq = 0.0f;
        if (race_ahead(o, t)) t = o;
    }
    __syncthreads();
    return t;
}

// Wave 0 finds, in a 256-bin count histogram read from the top bin down,
// the bin where the running count first reaches `need`; writes sel[0] = bin,
// sel[1] = count above it, sel[2] = its count.  Needs 1 <= need <= total.
__device__ __forceinline__ void wave0_find_bin(const uint32_t *hist, uint32_t need,
                                               uint32_t *sel) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
        uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
        uint32_t s = h0 + h1 + h2 + h3;
        // suffix sum over lanes >= lane: the total less the prefix before
        const uint32_t inc = wave_incl_scan_u32(s, lane);
        const uint32_t S = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63) - inc + s;
        uint32_t above = S - s;
        if (above < need && S >= need) {
            uint32_t acc = above, d, c;
            if (acc + h3 >= need) {
                d = 4 * lane + 3; c = h3;
            } else if (acc + h3 + h2 >= need) {
                acc += h3; d = 4 * lane + 2; c = h2;
            } else if (acc + h3 + h2 + h1 >= need) {
                acc += h3 + h2; d = 4 * lane + 1; c = h1;
            } else {
                acc += h3 + h2 + h1; d = 4 * lane; c = h0;
            }
            sel[0] = d;
            sel[1] = acc;
            sel[2] = c;
        }
    }
}

// Workgroup reduction of four 64-bit values at once: minimum, maximum, OR
// and AND (sc: 4 * NT / 64 entries).  Two barriers.
template <int NT>
__device__ __forceinline__ void wg_min_max_or_and(uint64_t &mn, uint64_t &mx, uint64_t &o,
                                                  uint64_t &a, uint64_t *sc) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const uint64_t x0 = xlane64(mn, m), x1 = xlane64(mx, m), x2 = xlane64(o, m), x3 = xlane64(a, m);
        mn = x0 < mn ? x0 : mn;
        mx = x1 > mx ? x1 : mx;
        o |= x2;
        a &= x3;
    }
    constexpr int NW = NT / 64;
    if ((threadIdx.x & 63) == 0) {
        const int w = threadIdx.x >> 6;
        sc[w] = mn;
        sc[NW + w] = mx;
        sc[2 * NW + w] = o;
        sc[3 * NW + w] = a;
    }
    __syncthreads();
    mn = ~0ull;
    mx = 0ull;
    o = 0ull;
    a = ~0ull;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        mn = sc[i] < mn ? sc[i] : mn;
        mx = sc[NW + i] > mx ? sc[NW + i] : mx;
        o |= sc[2 * NW + i];
        a &= sc[3 * NW + i];
    }
    __syncthreads();
}

// Radix select over distinct 64-bit composites held in registers.  Finds
// (prefix, pmask) such that exactly kk of the valid entries satisfy
// (v & pmask) >= prefix, i.e. the kk largest.  Digits of up to 8 bits are
// taken from the highest bit that differs among the entries down, skipping
// bits every entry shares (the low half of a bf16 value's key, the high bits
// of ids below V), and stopping as soon as the boundary bucket is taken
// whole.  Once only id bits remain, the bucket is a run of equal values: if
// it fits in tie[] (tcap entries of LDS), its members are ranked by direct
// comparison and the need-th largest becomes the exact boundary.  Needs
// 1 <= kk < number of valid entries.
template <int NT, int R>
__device__ __forceinline__ void wg_radix_select(const uint64_t (&v)[R], uint32_t vmask, uint32_t kk,
                                uint32_t *hist, uint32_t *sel, uint64_t *sc64, uint64_t *tie,
                                uint32_t tcap, uint32_t *tcnt, uint64_t &prefix_out,
                                uint64_t &pmask_out) {
    uint64_t mn = ~0ull, mx = 0ull, o = 0ull, an = ~0ull;
#pragma unroll
    for (int r = 0; r < R; ++r)
        if ((vmask >> r) & 1u) {
            mn = v[r] < mn ? v[r] : mn;
            mx = v[r] > mx ? v[r] : mx;
            o |= v[r];
            an &= v[r];
        }
    wg_min_max_or_and<NT>(mn, mx, o, an, sc64);
    const uint64_t vary = o ^ an;  // bits that differ somewhere
    if (vary == 0) {               // a single entry
        prefix_out = mx;
        pmask_out = ~0ull;
        return;
    }
    int hi = 63 - __clzll(vary);
    uint64_t pmask = (hi == 63) ? 0ull : (~0ull << (hi + 1));
    uint64_t prefix = mx & pmask;
    uint32_t need = kk;
    for (;;) {
        if (hi < 32) {
            // equal values from here on: rank the bucket's members directly
            uint32_t cnt = 0;
            if (threadIdx.x == 0) *tcnt = 0;
            __syncthreads();
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (((vmask >> r) & 1u) && (v[r] & pmask) == prefix) {
                    const uint32_t pos = atomicAdd(tcnt, 1u);
                    if (pos < tcap) tie[pos] = v[r];
                }
            __syncthreads();
            cnt = *tcnt;
            if (cnt <= tcap) {
                for (uint32_t i = threadIdx.x; i < cnt; i += NT) {
                    const uint64_t me = tie[i];
                    uint32_t above = 0;
                    for (uint32_t j2 = 0; j2 < cnt; ++j2) above += tie[j2] > me;
                    if (above == need - 1) sc64[0] = me;
                }
                __syncthreads();
                prefix = sc64[0];
                pmask = ~0ull;
                __syncthreads();
                break;
            }
            // a run of equal values larger than tie[]: id digits as below
        }
        const int width = hi + 1 < 8 ? hi + 1 : 8;
        const int shift = hi + 1 - width;
        const uint32_t dmask = (1u << width) - 1u;
        for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (((vmask >> r) & 1u) && (v[r] & pmask) == prefix)
                atomicAdd(&hist[(uint32_t)(v[r] >> shift) & dmask], 1u);
        __syncthreads();
        wave0_find_bin(hist, need, sel);
        __syncthreads();
        const uint32_t d = sel[0], above = sel[1], cntd = sel[2];
        need -= above;
        prefix |= (uint64_t)d << shift;
        pmask |= (uint64_t)dmask << shift;
        if (cntd == need || shift == 0) break;
        // next digit: from the highest bit below this one that differs
        // somewhere; the bits skipped are the same in every entry
        const uint64_t rest = vary & ((1ull << shift) - 1ull);
        if (rest == 0) break;  // cannot happen for distinct entries
        hi = 63 - __clzll(rest);
        const uint64_t skip = ((1ull << shift) - 1ull) & ~((1ull << (hi + 1)) - 1ull);
        pmask |= skip;
        prefix |= mx & skip;
    }
    prefix_out = prefix;
    pmask_out = pmask;
}

// Descending bitonic sort of s[0..n), n a power of two.  Callers barrier
// before; ends with a barrier.
template <int NT>
__device__ void bitonic_desc(uint64_t *s, int n) {
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < n; i += NT) {
                int ixj = i ^ j;
                if (ixj > i) {
                    uint64_t a = s[i], c = s[ixj];
                    bool desc = (i & k) == 0;
                    if (desc ? (a < c) : (a > c)) {
                        s[i] = c;
                        s[ixj] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
}

// Descending bitonic sort of npad <= K3_THREADS composites, one per thread
// (thread i holds place i afterwards): exchanges between lanes of a wave go
// by shuffles, wider ones through s[0..K3_THREADS) in LDS (a barrier
// pair each).  npad is a power of two; every thread of the workgroup calls.
__device__ uint64_t bitonic_regs_desc(uint64_t c, int npad, uint64_t *s) {
    const int tid = threadIdx.x;
    // a wave holding no place below npad only joins the barriers
    const bool busy = (tid & ~63) < npad;
    for (int k = 2; k <= npad; k <<= 1) {
        for (int j = k >> 1; j >= 64; j >>= 1) {
            s[tid] = c;
            __syncthreads();
            const uint64_t o = s[tid ^ j];
            __syncthreads();
            const bool lower = (tid & j) == 0;
            const bool desc = (tid & k) == 0;
            c = (lower == desc) ? (o > c ? o : c) : (o < c ? o : c);
        }
        if (busy) {
            // within the wave: constant lane masks (every lane active)
#pragma unroll
            for (int j = 32; j >= 1; j >>= 1)
                if (j < k) {
                    const uint64_t o = xlane64(c, j);
                    const bool lower = (tid & j) == 0;
                    const bool desc = (tid & k) == 0;
                    c = (lower == desc) ? (o > c ? o : c) : (o < c ? o : c);
                }
        }
    }
    return c;
}

__device__ __forceinline__ int pow2_ceil(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

// Chunk/segment-local bitmap of a row's history ids (duplicates collapse,
// ids outside [seg0, seg0 + len) ignored).  Begins and ends with barriers.
template <int NT>
__device__ __forceinline__ void build_bitmap(uint32_t *bm, int64_t seg0, int64_t len, const KParams &P, int b) {
    const int nw = (int)((len + 31) >> 5);
    __syncthreads();
    for (int w = threadIdx.x; w < nw; w += NT) bm[w] = 0u;
    __syncthreads();
    const int64_t i0 = P.offsets[b];
    int64_t i1 = P.offsets[b + 1];
    if (P.plen) {  // only the filled part of the slot is history
        const int64_t n = P.plen[b] < 0 ? 0 : P.plen[b];
        if (i0 + n < i1) i1 = i0 + n;
    }
    for (int64_t t = i0 + threadIdx.x; t < i1; t += NT) {
        int64_t r = (int64_t)P.ids[t] - seg0;
        if (r >= 0 && r < len) atomicOr(&bm[r >> 5], 1u << (r & 31));
    }
    __syncthreads();
}

__device__ __forceinline__ const void *row_ptr(const KParams &P, int dt, int b) {
    return (const char *)P.logits + (int64_t)b * P.ld * (dt == 1 ? 2 : 4);
}

// ================================================================== row helpers

__device__ __forceinline__ int group_nv(int j, int end) {
    const int rem = end - j;
    return rem <= 0 ? 0 : (rem >= 8 ? 8 : rem);
}

// Raw (not yet widened) registers of one group of 8 logits, so that the
// loads of the next batch can be in flight while the current one is used.
template <int DT>
struct Raw;
template <>
struct Raw<1> {
    u32x4 v;  // 8 bf16
};
template <>
struct Raw<0> {
    f32x4 a, b;  // 8 fp32
};

template <int DT, bool AL>
__device__ __forceinline__ void load_raw(const void *p, int64_t j, int nv, Raw<DT> &r) {
    if (DT == 1) {
        u32x4 &v = reinterpret_cast<Raw<1> &>(r).v;
        if (AL && nv == 8) {
            v = __builtin_nontemporal_load((const u32x4 *)((const uint16_t *)p + j));
        } else {
            const uint16_t *h = (const uint16_t *)p + j;
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t lo = (2 * i < nv) ? h[2 * i] : 0u;
                uint32_t hi = (2 * i + 1 < nv) ? h[2 * i + 1] : 0u;
                w[i] = lo | (hi << 16);
            }
            v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
        }
    } else {
        Raw<0> &f = reinterpret_cast<Raw<0> &>(r);
        if (AL && nv == 8) {
            const f32x4 *q = (const f32x4 *)((const float *)p + j);
            f.a = __builtin_nontemporal_load(q);
            f.b = __builtin_nontemporal_load(q + 1);
        } else {
            const float *q = (const float *)p + j;
            float t[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) t[i] = (i < nv) ? q[i] : 0.0f;
            f.a.x = t[0]; f.a.y = t[1]; f.a.z = t[2]; f.a.w = t[3];
            f.b.x = t[4]; f.b.y = t[5]; f.b.z = t[6]; f.b.w = t[7];
        }
    }
}

template <int DT>
__device__ __forceinline__ void unpack_raw(const Raw<DT> &r, float (&x)[8]) {
    if (DT == 1) {
        const u32x4 &u = reinterpret_cast<const Raw<1> &>(r).v;
        x[0] = __uint_as_float(u.x << 16);
        x[1] = __uint_as_float(u.x & 0xffff0000u);
        x[2] = __uint_as_float(u.y << 16);
        x[3] = __uint_as_float(u.y & 0xffff0000u);
        x[4] = __uint_as_float(u.z << 16);
        x[5] = __uint_as_float(u.z & 0xffff0000u);
        x[6] = __uint_as_float(u.w << 16);
        x[7] = __uint_as_float(u.w & 0xffff0000u);
    } else {
        const Raw<0> &f = reinterpret_cast<const Raw<0> &>(r);
        x[0] = f.a.x; x[1] = f.a.y; x[2] = f.a.z; x[3] = f.a.w;
        x[4] = f.b.x; x[5] = f.b.y; x[6] = f.b.z; x[7] = f.b.w;
    }
}

// Running (max, sum exp(x - max), finite min) of one thread.  Terms are
// hardware fp32 exponentials (exp2 of a scaled argument: relative error grows
// like |x - max| * 2^-24, so the mass-weighted error of the total stays near
// 1e-6 even for long flat tails), summed in fp32 per group of 8 (each term
// <= 1, so a group sum carries a few 1e-7 relative) and the group sums in
// double; when the running max rises
// the sum is rescaled by an fp32 exponential of the (non-positive)
// difference, a few times per chunk at most.
struct Stats {
    float m, xmin;
    double z;
};
template <int UU, int N = 8>
__device__ __forceinline__ void stats_batch(Stats &st, const float (&x)[UU][N], const int (&nv)[UU]) {
    float tm = -INFINITY;
#pragma unroll
    for (int u = 0; u < UU; ++u)
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < nv[u]) {
                tm = fmaxf(tm, x[u][i]);
                if (x[u][i] > -INFINITY) st.xmin = fminf(st.xmin, x[u][i]);
            }
    if (tm > st.m) {
        if (st.z != 0.0) st.z *= (double)expf(st.m - tm);
        st.m = tm;
    }
    if (st.m > -INFINITY) {
#pragma unroll
        for (int u = 0; u < UU; ++u) {
            float zs = 0.0f;
#pragma unroll
            for (int i = 0; i < N; ++i)
                if (i < nv[u]) zs += __expf(x[u][i] - st.m);
            st.z += (double)zs;
        }
    }
}

__device__ __forceinline__ ChunkStat empty_stat() {
    ChunkStat cs;
    cs.m = -INFINITY;
    cs.xmin = INFINITY;
    cs.z = 0.0;
    cs.rx = -INFINITY;
    cs.rqe = 1.0f;
    cs.ridx = NONE;
    cs.nstr = 0;
    return cs;
}

// ---------------------------------------------------------------- k_plan
// Per row, before the streaming pass: the admission estimate of rows with
// top-k or top-p (the value the pass filters their tiles with), and the
// transformed sample maximum, the reference the pass sums exponentials
// against.

struct StreamShared {
    uint64_t sc64[16];
    double scd[16];
    float scx[16], scq[16];
    uint32_t sci[16];
    uint32_t hist[256];
    uint32_t sel[4];
};

// Admission value t of a top-k / top-p row, chosen so that the row holds at
// least kk elements >= t with high probability, and not many more: close
// below the r-th largest raw logit of a sample -- EST_SEGS runs of EST_SEG
// elements, one in each of EST_SEGS equal segments of the row, or the whole
// row when it is shorter than EST_N -- r
// being the sample rank expected for the row's kk-th largest plus four
// standard deviations of it plus 8.  The sample's order keys are binned by
// their distance below the sample maximum in steps of 2^16 (one bf16 ulp);
// only the top 255 bins are counted, so the bins stay sparse and the LDS
// atomics rarely collide.  When those bins hold fewer than r keys (a few
// samples far above the rest stretch the range: spikes, or one large
// extreme value), the r-th key is found in two steps instead: its bin of
// 2^24 (256 fine steps), then its fine bin inside that one, so the value
// keeps the same resolution whatever the spread above it.  -inf (admit
// everything) when r would exceed the sample.
// smax receives the sample maximum (raw); active whether the row has top-k
// or top-p at all (the sample is requested before the row's stages are
// known, so that the two latencies overlap).
// Only the speed depends on t: the row merge checks that what the pass
// admitted holds the row's kk largest and sends the row to the full-row
// search when it does not.
// The sample runs (est_run_start) are staggered so that the runs of all
// rows do not start at the same offsets modulo a large power of two, where
// they would all fall on the same few memory channels.

template <int DT, bool AL>
__device__ __forceinline__ float row_estimate(const KParams &P, int b, StreamShared &S,
                                              float &smax, float &smin, bool &active) {
    constexpr int NT = K1_THREADS;
    constexpr int PER = EST_N / (NT * VEC);  // groups of 8 per thread
    constexpr int GPS = EST_SEG / VEC;       // groups per run
    const int V = P.V;
    const bool whole = V <= EST_N;
    const int n = whole ? V : EST_N;
    const void *rowp = row_ptr(P, DT, b);
    // the whole sample in registers, every load in flight at once
    Raw<DT> raw[PER];
    int nv[PER];
#pragma unroll
    for (int g = 0; g < PER; ++g) {
        const int gi = (int)threadIdx.x + g * NT;
        int j;
        if (whole) {
            j = gi * VEC;
        } else {
            const int seg = gi / GPS;
            j = est_run_start(seg, b, V) + (gi % GPS) * VEC;
        }
        nv[g] = group_nv(j, V);
        load_raw<DT, AL>(rowp, j, nv[g], raw[g]);
    }
    // the row's stages, read while the sample is on its way (rows without
    // top-k / top-p leave here, their sample unused)
    const Mode md = row_mode(P, b);
    active = md.tk || md.tp;
    if (!active) return 0.0f;
    const uint32_t kk = md.tk ? (uint32_t)md.k : (uint32_t)min(P.guess, P.V);
    const double r0 = (double)kk * (double)n / (double)V;
    const double rr = ceil(r0 + 4.0 * sqrt(r0) + 8.0);
    const uint32_t r = rr < (double)n ? (uint32_t)rr : 0u;  // 0: admit everything
    // the sample maximum and smallest finite value
    const uint32_t kninf = f2key(-INFINITY);
    uint32_t mx = 0, mn = ~0u;
#pragma unroll
    for (int g = 0; g < PER; ++g) {
        float x[8];
        unpack_raw<DT>(raw[g], x);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < nv[g]) {
                const uint32_t k = f2key(x[i]);
                mx = max(mx, k);
                if (k > kninf) mn = min(mn, k);
            }
    }
#pragma unroll
    for (int sft = 32; sft >= 1; sft >>= 1) {
        mx = max(mx, shx(mx, sft));
        mn = min(mn, shx(mn, sft));
    }
    if ((threadIdx.x & 63) == 0) {
        S.sci[threadIdx.x >> 6] = mx;
        S.sci[8 + (threadIdx.x >> 6)] = mn;
    }
    __syncthreads();
    mx = S.sci[0];
    mn = S.sci[8];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) {
        mx = max(mx, S.sci[i]);
        mn = min(mn, S.sci[8 + i]);
    }
    smax = key2f(mx);
    smin = mn == ~0u ? INFINITY : key2f(mn);
    if (r == 0) return -INFINITY;
    // histogram of the keys whose distance below the maximum, in steps of
    // 2^shift and counted from `base` steps, is below `nb`; bin 255 - d
    // holds distance base + d.  Returns the number of keys counted.
    auto fill = [&](int shift, uint32_t base, uint32_t nb) -> uint32_t {
        for (int i = threadIdx.x; i < 256; i += NT) S.hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int g = 0; g < PER; ++g) {
            float x[8];
            unpack_raw<DT>(raw[g], x);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t d = ((mx - f2key(x[i])) >> shift) - base;
                if (i < nv[g] && d < nb) atomicAdd(&S.hist[255 - d], 1u);
            }
        }
        __syncthreads();
        if (threadIdx.x < 64) {
            uint32_t tot = S.hist[4 * threadIdx.x] + S.hist[4 * threadIdx.x + 1] +
                           S.hist[4 * threadIdx.x + 2] + S.hist[4 * threadIdx.x + 3];
#pragma unroll
            for (int sft = 32; sft >= 1; sft >>= 1) tot += shx(tot, sft);
            if (threadIdx.x == 0) S.sel[3] = tot;
        }
        __syncthreads();
        return S.sel[3];
    };
    // the fine bin (distance from the maximum, in steps of 2^16) holding the
    // need-th largest key of the histogram just filled, given `base`
    auto pick = [&](uint32_t need, uint32_t base) -> float {
        wave0_find_bin(S.hist, need, S.sel);
        __syncthreads();
        const uint32_t d = base + (255u - S.sel[0]);
        // every key of fine bins 0..d, i.e. key > mx - (d + 1) * 2^16
        const uint64_t lo = (uint64_t)mx - (((uint64_t)d + 1) << 16) + 1;
        const uint32_t fk = lo > (uint64_t)mx ? 0u : (uint32_t)lo;
        return fk <= f2key(-INFINITY) ? -INFINITY : key2f(fk);
    };
    if (fill(16, 0u, 255u) >= r) return pick(r, 0u);
    // spread-out top: the coarse bin of the r-th key, then its fine bin
    if (fill(24, 0u, 255u) < r) return -INFINITY;  // unreachable: 255 * 2^24 spans every key
    wave0_find_bin(S.hist, r, S.sel);
    __syncthreads();
    const uint32_t dc = 255u - S.sel[0];
    const uint32_t above = S.sel[1];
    __syncthreads();
    (void)fill(16, dc << 8, 256u);
    return pick(r - above, dc << 8);
}

// One workgroup per row, before the pass: for rows with top-k or top-p, the
// admission estimate and the reference of the exponential sums.
template <int DT, bool AL, bool XF>
__global__ __launch_bounds__(K1_THREADS) void k_plan(KParams P, KPlan L, KWork W) {
    __shared__ StreamShared S;
    const int b = P.b0 + (int)blockIdx.x;
    float smax, smin;
    bool active;
    const float t = row_estimate<DT, AL>(P, b, S, smax, smin, active);
    if (!active) return;
    if (threadIdx.x == 0) {
        W.rowthr[b] = t;
        W.rowref[b] = xform<XF>(smax, 0u, P);
        W.rowlo[b] = smin < INFINITY ? xform<XF>(smin, 0u, P) : INFINITY;
    }
}

// ---------------------------------------------------------------- k_pass
// The one streaming pass over the logits: one workgroup per tile of
// L.seg elements (the segment length v of the Ascend page's rolling top-k by
// default), every tile of every row in one grid, so the hardware dispatcher
// spreads rows of every kind over all CUs.  Each thread keeps pass_depth
// groups of its share of the tile in flight (the whole share of an fp32 tile
// of 8192): groups of 4 consecutive elements, one 16-byte streaming store per
// group of dense output, consecutive lanes on consecutive groups.
//  * rows without top-k / top-p: the dense output gets the transformed
//    logits; the exponential race over the tile runs with q read in the same
//    pass, or the greedy argmax; optional statistics for the probabilities;
//  * rows with top-k or top-p: admission against the row's estimate (see
//    row_estimate), each wave appending to its own sub-slot, and statistics
//    for rows without top-k; their dense output is written once the kept
//    set is known (k_dense), in whole lines.  A wave whose admissions exceed
//    its sub-slot (L.wcap) marks it overflowed; the row merge then sends the
//    row to the full-row search.

constexpr int PASS_THREADS = 256;
constexpr int PASS_WAVES = PASS_THREADS / 64;
// Groups of 4 in flight per thread in the pass: 8 for fp32 logits (16
// bytes a group), 6 for bf16 (8 bytes a group), whose fewer registers let
// more waves share a CU.
template <int DT>
constexpr int pass_depth() { return DT == 1 ? 6 : 8; }
constexpr int PASS_D_MAX = 8;
static_assert(pass_depth<0>() <= PASS_D_MAX && pass_depth<1>() <= PASS_D_MAX,
              "a lane's admissions of a chunk are one bit each of a 32-bit mask (4 per group)");
constexpr int PGROUP = PASS_THREADS * 4;       // elements per group row

template <int DT>
struct Raw4;
template <>
struct Raw4<1> {
    u32x2 v;  // 4 bf16
};
template <>
struct Raw4<0> {
    f32x4 v;  // 4 fp32
};

__device__ __forceinline__ int nv4(int j, int end) {
    const int rem = end - j;
    return rem <= 0 ? 0 : (rem >= 4 ? 4 : rem);
}

template <int DT, bool AL>
__device__ __forceinline__ void load4(const void *p, int j, int nv, Raw4<DT> &r) {
    if (DT == 1) {
        u32x2 &v = reinterpret_cast<Raw4<1> &>(r).v;
        if (AL && nv == 4) {
            v = __builtin_nontemporal_load((const u32x2 *)((const uint16_t *)p + j));
        } else {
            const uint16_t *h = (const uint16_t *)p + j;
            uint32_t w[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint32_t lo = (2 * i < nv) ? h[2 * i] : 0u;
                const uint32_t hi = (2 * i + 1 < nv) ? h[2 * i + 1] : 0u;
                w[i] = lo | (hi << 16);
            }
            v.x = w[0];
            v.y = w[1];
        }
    } else {
        f32x4 &v = reinterpret_cast<Raw4<0> &>(r).v;
        if (AL && nv == 4) {
            v = __builtin_nontemporal_load((const f32x4 *)((const float *)p + j));
        } else {
            const float *q = (const float *)p + j;
            v.x = nv > 0 ? q[0] : 0.0f;
            v.y = nv > 1 ? q[1] : 0.0f;
            v.z = nv > 2 ? q[2] : 0.0f;
            v.w = nv > 3 ? q[3] : 0.0f;
        }
    }
}

template <int DT>
__device__ __forceinline__ void unpack4(const Raw4<DT> &r, float (&x)[4]) {
    if (DT == 1) {
        const u32x2 &u = reinterpret_cast<const Raw4<1> &>(r).v;
        x[0] = __uint_as_float(u.x << 16);
        x[1] = __uint_as_float(u.x & 0xffff0000u);
        x[2] = __uint_as_float(u.y << 16);
        x[3] = __uint_as_float(u.y & 0xffff0000u);
    } else {
        const f32x4 &v = reinterpret_cast<const Raw4<0> &>(r).v;
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
}

// Stores of 16 bytes per lane; the lanes of a wave write consecutive
// vectors, so a wave's store covers whole lines.  NT: streaming
// (non-temporal) stores, for the pass, whose dense output is written once
// and not read again; its write-back lines would otherwise still be draining
// into HBM while the next kernels run.  The dense writer keeps write-back
// stores, which it issues faster.
template <bool AL, bool NT = false>
__device__ __forceinline__ void store4(float *p, int j, int nv, const float (&x)[4]) {
    if (AL && nv == 4) {
        const f32x4 v = {x[0], x[1], x[2], x[3]};
        if (NT)
            __builtin_nontemporal_store(v, (f32x4 *)(p + j));
        else
            *(f32x4 *)(p + j) = v;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (i < nv) p[j + i] = x[i];
    }
}

// Penalty bits of the 4 elements starting at tile-relative offset r (a
// multiple of 4).
template <bool XF>
__device__ __forceinline__ uint32_t pen_bits4(const uint32_t *bm, int r, const KParams &P) {
    if (!XF || !P.pen) return 0u;
    return (bm[r >> 5] >> (r & 31)) & 0xfu;
}

// Rank of this lane among the lanes set in a wave ballot.
__device__ __forceinline__ uint32_t lane_rank(uint64_t bal) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

// ---- wave-level reductions (every lane gets the result)
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shxf(v, m));
    return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += shxd(v, m);
    return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += shx(v, m);
    return v;
}
__device__ __forceinline__ Race wave_race(Race r) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        Race o;
        o.x = shxf(r.x, m);
        o.qe = shxf(r.qe, m);
        o.idx = shx(r.idx, m);
        o.lq = 0.0f;
        if (race_ahead(o, r)) r = o;
    }
    return r;
}

struct StreamState {
    Stats st;
    Race rc;
    float bx;     // greedy: this lane's largest value
    uint32_t bj;  // greedy: its lowest id (this lane's ids increase)
};

// Sum of exp(y - ref) for a select tile of a row without top-k: fp32 terms
// (the hardware exp2 of an exactly computed difference) against the row's
// reference (the transformed sample maximum), summed in fp32 over a lane's
// share and in double over the wave.  A wave that meets a value more than 64
// above the reference sums its share again against its own maximum.
struct RefSum {
    float z;     // sum of exp(y - ref)
    float ymax;  // largest y seen
};

// What a wave of a select tile has collected so far.
struct WaveSel {
    uint32_t cnt;     // entries handed over so far (uniform over the wave)
    bool ovf;         // the admissions did not fit the sub-slot
    uint32_t mask;    // this lane's admitted elements of the current chunk:
                      // bit 4 d + i = element i of its group in ring slot d
    uint32_t strict;  // this lane's handed-over entries above the estimate
};

// One group of 4 (first id j, nv valid, ring slot d) of a select tile: admit
// non-penalised elements with raw x >= traw and penalised ones (and, for
// rows that accumulate statistics, all of them) with transformed y >= yt,
// where yt is the transform of traw; every element left out therefore has
// y <= yt.  The admitted elements only set bits of the lane's mask; a lane
// that admits any keeps the raw group in its LDS staging slot, where the
// chunk's compaction reads it back.
template <int DT, bool XF, bool FULL, bool STATS>
__device__ __forceinline__ void sel_group(const Raw4<DT> &raw, int j, int nv, int c0, int d,
                                          const uint32_t *bm, const KParams &P, RefSum &rs,
                                          WaveSel &ws, Raw4<DT> *stage, float ref, float traw,
                                          float yt) {
    float x[4];
    unpack4<DT>(raw, x);
    const uint32_t bits = (FULL || nv > 0) ? pen_bits4<XF>(bm, j - c0, P) : 0u;
    bool c[4];
    if (STATS) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float y = xform<XF>(x[i], (bits >> i) & 1u, P);
            if (FULL || i < nv) {
                rs.ymax = fmaxf(rs.ymax, y);
                rs.z += __builtin_amdgcn_exp2f((y - ref) * 1.4426950408889634f);
            }
            c[i] = (FULL || i < nv) && y >= yt;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = (FULL || i < nv) && x[i] >= traw;
        if (XF && bits) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if ((bits >> i) & 1u) c[i] = (FULL || i < nv) && xform<XF>(x[i], 1u, P) >= yt;
        }
    }
    const uint32_t cb = (uint32_t)c[0] | ((uint32_t)c[1] << 1) | ((uint32_t)c[2] << 2) |
                        ((uint32_t)c[3] << 3);
    if (cb) {
        stage[d * 64 + (threadIdx.x & 63)] = raw;
        ws.mask |= cb << (4 * d);
    }
}

// Hand over a chunk's admitted elements: each lane's place in the wave's
// sub-slot is the exclusive prefix of the lanes' counts (at most 32, so six
// ballots of bit planes give it), and each lane then writes its entries,
// reading their raw values back from its staging slots.  jd is the first id
// of the lane's group in ring slot 0.
template <int DT, bool XF>
__device__ __forceinline__ void sel_compact(WaveSel &ws, const Raw4<DT> *stage, int jd, int c0,
                                            const uint32_t *bm, const KParams &P, uint64_t *dst,
                                            uint32_t wcap, float yt) {
    uint32_t mask = ws.mask;
    ws.mask = 0;
    const uint32_t n = (uint32_t)__popc(mask);
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
        const uint64_t bal = __ballot((n >> bit) & 1u);
        pre += lane_rank(bal) << bit;
        tot += (uint32_t)__popcll(bal) << bit;
    }
    if (tot == 0) return;
    if (ws.ovf || ws.cnt + tot > wcap) {
        ws.ovf = true;
        return;
    }
    uint32_t off = ws.cnt + pre;
    const int lane = threadIdx.x & 63;
    while (mask) {
        const uint32_t e = (uint32_t)__ffs(mask) - 1u;
        mask &= mask - 1u;
        const uint32_t d = e >> 2, i = e & 3u;
        float x;
        if (DT == 1) {
            const uint16_t *h = reinterpret_cast<const uint16_t *>(stage + d * 64 + lane);
            x = __uint_as_float((uint32_t)h[i] << 16);
        } else {
            x = reinterpret_cast<const float *>(stage + d * 64 + lane)[i];
        }
        const int j = jd + (int)d * PGROUP + (int)i;
        uint32_t pb = 0;
        if (XF && P.pen) {
            const int r = j - c0;
            pb = (bm[r >> 5] >> (r & 31)) & 1u;
        }
        const float y = xform<XF>(x, pb, P);
        dst[off++] = mkcomp(y, (uint32_t)j);
        ws.strict += y > yt;
    }
    ws.cnt += tot;
}

// One group of 4 of a row without top-k / top-p: transform, dense store,
// statistics, and the race (q given) or the greedy argmax.
template <int DT, bool AL, bool XF, bool FULL, bool STATS, bool RACE>
__device__ __forceinline__ void stream_group(const Raw4<DT> &raw, const Raw4<0> &qraw, int j, int nv,
                                             int c0, const uint32_t *bm, const KParams &P,
                                             float *rowo, StreamState &ss) {
    float y[1][4];
    unpack4<DT>(raw, y[0]);
    const uint32_t bits = (FULL || nv > 0) ? pen_bits4<XF>(bm, j - c0, P) : 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[0][i] = xform<XF>(y[0][i], (bits >> i) & 1u, P);
    if (rowo && (FULL || nv > 0)) store4<AL, true>(rowo, j, FULL ? 4 : nv, y[0]);
    if (STATS) {
        int nvv[1] = {FULL ? 4 : nv};
        stats_batch<1, 4>(ss.st, y, nvv);
    }
    if (RACE) {
        float qv[4];
        unpack4<0>(qraw, qv);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (FULL || i < nv) race_offer(ss.rc, y[0][i], qv[i] + P.eps, (uint32_t)(j + i));
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if ((FULL || i < nv) && y[0][i] > ss.bx) {
                ss.bx = y[0][i];
                ss.bj = (uint32_t)(j + i);
            }
    }
}

// Sum of exp(y - m) over this lane's groups of the tile [c0, c1), read
// again (rare path: a value far above the row's reference).
template <int DT, bool AL, bool XF>
__device__ __forceinline__ double lane_sum_again(const KParams &P, const uint32_t *bm, int b, int c0, int c1,
                                 float m) {
    const void *rowp = row_ptr(P, DT, b);
    double z = 0.0;
    for (int j = c0 + (int)threadIdx.x * 4; j < c1; j += PGROUP) {
        const int nv = nv4(j, c1);
        Raw4<DT> raw;
        load4<DT, AL>(rowp, j, nv, raw);
        float x[4];
        unpack4<DT>(raw, x);
        const uint32_t bits = pen_bits4<XF>(bm, j - c0, P);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (i < nv) z += (double)__expf(xform<XF>(x[i], (bits >> i) & 1u, P) - m);
    }
    return z;
}

// The group loop of a tile: pass_depth<DT>() groups in flight per thread (q for racing
// rows QD groups ahead), each group processed as soon as it arrives.
template <int DT, bool AL, bool XF, int KIND, bool FULL, bool STATS>
__device__ __forceinline__ void tile_loop(const uint32_t *bm, const KParams &P, int c0, int c1,
                                          int ng, int j0, const void *rowp, const float *rowq,
                                          float *rowo, Raw4<DT> (&ring)[pass_depth<DT>()], StreamState &ss,
                                          RefSum &rs, WaveSel &ws, Raw4<DT> *stage, uint64_t *dst,
                                          uint32_t wcap, float ref, float traw, float yt) {
    constexpr int PASS_D = pass_depth<DT>();
    constexpr int QD = KIND == 1 ? PASS_D / 2 : 1;
    Raw4<0> qring[QD];
    if (KIND == 1) {
#pragma unroll
        for (int d = 0; d < QD; ++d)
            if (d < ng) {
                const int j = j0 + d * PGROUP;
                const int nv = FULL ? 4 : nv4(j, c1);
                if (nv > 0) load4<0, AL>(rowq, j, nv, qring[d]);
            }
    }
    for (int g0 = 0; g0 < ng; g0 += PASS_D) {
#pragma unroll
        for (int d = 0; d < PASS_D; ++d) {
            const int g = g0 + d;
            if (g < ng) {
                const int j = j0 + g * PGROUP;
                const int nv = FULL ? 4 : nv4(j, c1);
                if (KIND == 2)
                    sel_group<DT, XF, FULL, STATS>(ring[d], j, nv, c0, d, bm, P, rs, ws, stage,
                                                   ref, traw, yt);
                else
                    stream_group<DT, AL, XF, FULL, STATS, KIND == 1>(ring[d], qring[d % QD], j, nv,
                                                                     c0, bm, P, rowo, ss);
                const int gn = g + PASS_D;
                if (gn < ng) {
                    const int jn = j0 + gn * PGROUP;
                    const int nvn = FULL ? 4 : nv4(jn, c1);
                    if (nvn > 0) load4<DT, AL>(rowp, jn, nvn, ring[d]);
                }
                if (KIND == 1 && g + QD < ng) {
                    const int jq = j0 + (g + QD) * PGROUP;
                    const int nvq = FULL ? 4 : nv4(jq, c1);
                    if (nvq > 0) load4<0, AL>(rowq, jq, nvq, qring[d % QD]);
                }
            }
        }
        // the chunk's admissions go out while the next chunk is on its way
        if (KIND == 2) sel_compact<DT, XF>(ws, stage, j0 + g0 * PGROUP, c0, bm, P, dst, wcap, yt);
    }
}

// One tile, each wave on its own: no barrier (the penalty bitmap aside).
// Wave w of tile t of row b collects its candidates in its own LDS buffer
// (appends to global memory in the middle of the load stream would make the
// wave wait for its stores), hands them over in sub-slot t * PASS_WAVES + w
// of the row at the end, and writes its statistics / winner to the same
// entry of the row's wave records.
template <int DT, bool AL, bool XF, int KIND>
__device__ __forceinline__ void pass_tile(const uint32_t *bm, const KParams &P, const KPlan &L,
                                          const KWork &W, const Mode &md, int b, int t,
                                          float traw, float ref, Raw4<DT> (&ring)[pass_depth<DT>()],
                                          Raw4<DT> *stage) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int c0 = t * L.seg;
    const int c1 = min(c0 + L.seg, P.V);
    const int ng = (c1 - c0 + PGROUP - 1) / PGROUP;  // group rows in the tile
    const bool full = c0 + ng * PGROUP <= c1;        // every group whole
    const void *rowp = row_ptr(P, DT, b);
    const float *rowq = KIND == 1 ? P.q + (int64_t)b * P.V : nullptr;
    // the pass writes the dense output of unfiltered rows; filtered rows get
    // theirs from the dense writer once their kept sets are known
    float *rowo = (KIND != 2 && P.out_logits) ? P.out_logits + (int64_t)b * P.V : nullptr;
    const bool do_stats = KIND == 2 ? !md.tk : (P.flags & NEED_PROBS) != 0;
    const int j0 = c0 + tid * 4;
    const int wslot = (b * L.nt + t) * PASS_WAVES + (tid >> 6);
    const uint32_t wcap = (uint32_t)L.wcap;
    Raw4<DT> *wstage = stage ? stage + (tid >> 6) * (pass_depth<DT>() * 64) : nullptr;
    uint64_t *dst = W.cand + (int64_t)b * ROWCAP + (int64_t)(t * PASS_WAVES + (tid >> 6)) * wcap;
    const float yt = KIND == 2 ? xform<XF>(traw, 0u, P) : 0.0f;
    StreamState ss;
    ss.st.m = -INFINITY; ss.st.xmin = INFINITY; ss.st.z = 0.0;
    ss.rc.x = -INFINITY; ss.rc.qe = 1.0f; ss.rc.idx = NONE; ss.rc.lq = 0.0f;
    ss.bx = -INFINITY;
    ss.bj = j0 < c1 ? (uint32_t)j0 : NONE;  // kept if every value is -inf
    RefSum rs;
    rs.z = 0.0f;
    rs.ymax = -INFINITY;
    WaveSel ws;
    ws.cnt = 0;
    ws.ovf = false;
    ws.mask = 0;
    ws.strict = 0;
#define SMP_TILE_LOOP(F, ST)                                                                    \
    tile_loop<DT, AL, XF, KIND, F, ST>(bm, P, c0, c1, ng, j0, rowp, rowq, rowo, ring, ss, rs, ws, \
                                       wstage, dst, wcap, ref, traw, yt)
    if (full) {
        if (do_stats) SMP_TILE_LOOP(true, true);
        else SMP_TILE_LOOP(true, false);
    } else {
        if (do_stats) SMP_TILE_LOOP(false, true);
        else SMP_TILE_LOOP(false, false);
    }
#undef SMP_TILE_LOOP
    ChunkStat cs = empty_stat();
    if (KIND == 2) {
        if (do_stats) {
            const float ym = wave_max_f32(rs.ymax);
            if (ym > ref + 64.0f) {
                cs.m = ym;
                cs.z = wave_sum_f64(lane_sum_again<DT, AL, XF>(P, bm, b, c0, c1, ym));
            } else {
                cs.m = ref;
                cs.z = wave_sum_f64((double)rs.z);
            }
        }
        // the entries went out chunk by chunk; count those above yt
        const uint32_t strict = wave_sum_u32(ws.strict);
        if (lane == 0) {
            W.wcnt[wslot] = ws.ovf ? 0xffffffffu : (ws.cnt | (strict << 16));
            W.cstat[wslot] = cs;
        }
    } else {
        if (do_stats) {
            const float M = wave_max_f32(ss.st.m);
            const double z = (ss.st.z != 0.0) ? ss.st.z * exp((double)ss.st.m - (double)M) : 0.0;
            cs.m = M;
            cs.z = wave_sum_f64(z);
        }
        if (KIND == 1) {
            const Race r = wave_race(ss.rc);
            cs.rx = r.x;
            cs.rqe = r.qe;
            cs.ridx = r.idx;
        } else {
            // the greedy winner: the largest value, lowest id among equals
            const float m = wave_max_f32(ss.bx);
            uint32_t id = (ss.bx == m) ? ss.bj : NONE;
#pragma unroll
            for (int sft = 32; sft >= 1; sft >>= 1) id = min(id, shx(id, sft));
            cs.rx = m;
            cs.rqe = 1.0f;
            cs.ridx = id;
        }
        if (lane == 0) W.cstat[wslot] = cs;
    }
}

template <int DT, bool AL, bool XF>
__global__ __launch_bounds__(PASS_THREADS) void k_pass(KParams P, KPlan L, KWork W) {
    // each wave's staging slots: the raw groups in which a lane admitted
    // something, read back when the chunk is handed over
    constexpr int PASS_D = pass_depth<DT>();
    __shared__ Raw4<DT> stage[PASS_WAVES][PASS_D * 64];
    extern __shared__ uint32_t bm[];  // penalty bitmap of the tile
    const int b = P.b0 + (int)(blockIdx.x / L.nt), t = (int)(blockIdx.x % L.nt);
    const int c0 = t * L.seg;
    const int c1 = min(c0 + L.seg, P.V);
    const int ng = (c1 - c0 + PGROUP - 1) / PGROUP;
    // the tile's logits are requested before anything about the row
    const void *rowp = row_ptr(P, DT, b);
    const int j0 = c0 + (int)threadIdx.x * 4;
    Raw4<DT> ring[PASS_D];
#pragma unroll
    for (int d = 0; d < PASS_D; ++d)
        if (d < ng) {
            const int j = j0 + d * PGROUP;
            const int nv = nv4(j, c1);
            if (nv > 0) load4<DT, AL>(rowp, j, nv, ring[d]);
        }
    const Mode md = row_mode(P, b);
    if (b == 0 && t == 0) {
        // the full-row search queue and its rows' synchronisation records
        if (threadIdx.x == 0) *W.fbcnt = 0u;
        for (int i = threadIdx.x; i < FB_GRID * FB_SYNC_WORDS; i += PASS_THREADS) W.fbsync[i] = 0u;
    }
    const bool filtering = P.top_k || P.top_p;  // the planning kernel ran
    const float traw = filtering ? W.rowthr[b] : 0.0f;
    const float ref = filtering ? W.rowref[b] : 0.0f;
    if (XF && P.pen) build_bitmap<PASS_THREADS>(bm, c0, c1 - c0, P, b);
    Raw4<DT> *st = &stage[0][0];
    if (md.tk || md.tp)
        pass_tile<DT, AL, XF, 2>(bm, P, L, W, md, b, t, traw, ref, ring, st);
    else if (md.sm)
        pass_tile<DT, AL, XF, 1>(bm, P, L, W, md, b, t, traw, ref, ring, st);
    else
        pass_tile<DT, AL, XF, 0>(bm, P, L, W, md, b, t, traw, ref, ring, st);
}

// Dense tiles (see k_dense and dense_tile), used by the row merge to group
// its kept list.
constexpr int DENSE_THREADS = 256;
static_assert(DGR == DENSE_THREADS * VEC, "a group-row is one group of 8 per lane");

// ================================================================== k_rows
// Per row, one workgroup of ROWS_THREADS: the exact kk largest of the row's
// candidates (held in registers, radix select), ordered only as far as top-p
// needs; fp64 softmax and prefix masses; the top-p cutoff (the top-k guess of
// the Ascend page's topP section is accepted only with a safe margin); the
// exponential race over K with q gathered by id, or the greedy pick; the
// kept list for the dense writer.  Rows without top-k / top-p merge their
// tiles' race or argmax winners.

constexpr int ROWS_THREADS = 256;

constexpr int RCAP = 4096;       // candidates held in registers by the merge
constexpr int NUC_STEPS = 16;    // top-p prefixes found without a sort, at most
constexpr int WAVE_TOPP = 256;   // selections this small: top-p by one wave, in registers
constexpr int WAVE_NUC = 4;      // maxima the wave looks at before it sorts (fixed: 4)

// 2^(j/64), j = 0..63: the table of exp_neg_tab, copied to LDS by the
// kernels that use it
__device__ const double exp2_j64_tab[64] = {SMP_EXP2_J64_VALUES};

struct RowsShared {
    double etab[64];          // exp2_j64_tab
    uint32_t addr[RCAP];      // slot address of each candidate (in-register path)
    uint64_t srt[KMAX];       // the kk selected
    uint64_t nuc[NUC_STEPS];  // a short top-p prefix, in order
    uint32_t hist[256];
    uint32_t sel[4];
    uint32_t sc[16];
    uint64_t sc64[16];
    double scd[16];
    float scx[16], scq[16];
    uint32_t sci[16];
    uint32_t cnt;
    double fd[2];
};

__device__ __forceinline__ void cx_desc(uint64_t &a, uint64_t &b) {
    const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
    a = hi;
    b = lo;
}
// The 4 largest of the 256 keys one wave holds (4 per lane), in descending
// order, in every lane: each lane sorts its own 4, then 6 exchange steps
// merge two sorted lists of 4 and keep the larger half (compare position i
// with the partner's position 3 - i, then sort the bitonic result).
__device__ __forceinline__ void wave_top4(const uint64_t (&v)[4], uint64_t (&t)[4]) {
    t[0] = v[0]; t[1] = v[1]; t[2] = v[2]; t[3] = v[3];
    cx_desc(t[0], t[1]);
    cx_desc(t[2], t[3]);
    cx_desc(t[0], t[2]);
    cx_desc(t[1], t[3]);
    cx_desc(t[1], t[2]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = xlane64(t[i], m);
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = t[i] > o[3 - i] ? t[i] : o[3 - i];
        cx_desc(t[0], t[2]);
        cx_desc(t[1], t[3]);
        cx_desc(t[0], t[1]);
        cx_desc(t[2], t[3]);
    }
}

// Descending bitonic sort of 256 keys held by one wave, key 4 lane + r in
// v[r]: partners in the same lane swap registers, partners in other lanes
// are exchanged with shuffles.  No LDS and no barrier.
__device__ __forceinline__ void wave_bitonic_desc256(uint64_t (&v)[4]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 2; k <= 256; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j >= 1; j >>= 1) {
            if (j >= 4) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int e = 4 * lane + r;
                    const uint64_t o = xlane64(v[r], j >> 2);
                    // in a descending block the lower index keeps the larger key
                    const bool keep_max = ((e & k) == 0) == ((e & j) == 0);
                    v[r] = keep_max ? (o > v[r] ? o : v[r]) : (o < v[r] ? o : v[r]);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int rp = r ^ j;
                    if (rp > r) {
                        const bool desc = ((4 * lane + r) & k) == 0;
                        const uint64_t a = v[r], c = v[rp];
                        if (desc ? (c > a) : (c < a)) {
                            v[r] = c;
                            v[rp] = a;
                        }
                    }
                }
            }
        }
    }
}

template <int NT>
__device__ __forceinline__ uint32_t wg_best_ratio(double r, uint32_t idx, double *scd,
                                                  uint32_t *sci) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        double ro = xlaned(r, m);
        uint32_t io = xlane(idx, m);
        if (ro > r || (ro == r && io < idx)) {
            r = ro;
            idx = io;
        }
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        scd[w] = r;
        sci[w] = idx;
    }
    __syncthreads();
    double br = scd[0];
    uint32_t bi = sci[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i)
        if (scd[i] > br || (scd[i] == br && sci[i] < bi)) {
            br = scd[i];
            bi = sci[i];
        }
    __syncthreads();
    return bi;
}

// Radix select over n distinct composites read by get(i), i < n (1 <= kk <
// n): (prefix, pmask) such that exactly kk of them satisfy (v & pmask) >=
// prefix.  Common high bits are skipped, then digits of up to 8 bits.
template <int NT, class G>
__device__ __forceinline__ void radix_select_any(uint32_t n, uint32_t kk, G &&get, uint32_t *hist, uint32_t *sel,
                                 uint64_t *sc64, uint64_t &prefix_out, uint64_t &pmask_out) {
    uint64_t mn = ~0ull, mx = 0ull;
    for (uint32_t i = threadIdx.x; i < n; i += NT) {
        const uint64_t v = get(i);
        mn = v < mn ? v : mn;
        mx = v > mx ? v : mx;
    }
    mn = wg_min_u64<NT>(mn, sc64);
    mx = wg_max_u64<NT>(mx, sc64);
    const uint64_t diff = mn ^ mx;
    if (diff == 0) {
        prefix_out = mx;
        pmask_out = ~0ull;
        return;
    }
    int hib = 63 - __clzll(diff);
    uint64_t pmask = (hib == 63) ? 0ull : (~0ull << (hib + 1));
    uint64_t prefix = mx & pmask;
    uint32_t need = kk;
    for (;;) {
        const int width = hib + 1 < 8 ? hib + 1 : 8;
        const int shift = hib + 1 - width;
        const uint32_t dmask = (1u << width) - 1u;
        for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0;
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < n; i += NT) {
            const uint64_t v = get(i);
            if ((v & pmask) == prefix) atomicAdd(&hist[(uint32_t)(v >> shift) & dmask], 1u);
        }
        __syncthreads();
        wave0_find_bin(hist, need, sel);
        __syncthreads();
        const uint32_t d = sel[0], above = sel[1], cntd = sel[2];
        __syncthreads();
        need -= above;
        prefix |= (uint64_t)d << shift;
        pmask |= (uint64_t)dmask << shift;
        if (cntd == need || shift == 0) break;
        hib = shift - 1;
    }
    prefix_out = prefix;
    pmask_out = pmask;
}

// Inverse-CDF position over a[0..n), n <= 4 NT, in the row's order (largest
// first): the least position whose inclusive mass sum of exp(x - x0) reaches
// u times the total; 0 when u <= 0 or NaN, n - 1 when rounding leaves the
// total short of the target.  Every thread returns it.
template <int NT>
__device__ __forceinline__ uint32_t inverse_cdf_pos(const uint64_t *a, uint32_t n, float x0, float u, double *scd,
                                    uint32_t *sc, const double *etab) {
    if (!(u > 0.0f) || n <= 1) return 0u;
    double e[4];
    double loc = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t p = 4 * threadIdx.x + i;
        e[i] = p < n ? exp_neg_tab((double)cval(a[p]) - (double)x0, etab) : 0.0;
        loc += e[i];
    }
    double tot;
    double run = wg_excl_scan_f64<NT>(loc, scd, tot);
    const double target = (double)u * tot;
    uint32_t first = NONE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t p = 4 * threadIdx.x + i;
        run += e[i];
        if (p < n && first == NONE && run >= target) first = p;
    }
    first = wg_min_u32<NT>(first, sc);
    return first == NONE ? n - 1 : first;
}

// The merge of an unfiltered row b (no top-k / top-p): its waves' maxima,
// minima and sums of exponentials, and their race winners (by ratio, lowest
// id on a tie) or argmax winners (by value, lowest id), over NT threads.
// Writes the output id and the row's info; queues an inverse-CDF draw over
// the whole row for the full-row search.  Scratch: 16 entries each.
template <int NT>
__device__ __forceinline__ void merge_unfiltered(const KParams &P, const KPlan &L, const KWork &W, int b,
                                 const Mode &md, double *scd, uint64_t *sc64, float *scx,
                                 float *scq, uint32_t *sci, const double *etab) {
    static_assert(NT / 64 <= 16, "scratch of 16 entries");
    const int tid = threadIdx.x;
    const int nt = L.nt * PASS_WAVES;  // wave records (sub-slots) of the row
    const ChunkStat *cst = W.cstat + (int64_t)b * nt;
    float m_loc = -INFINITY, mn_loc = INFINITY;
    for (int t = tid; t < nt; t += NT) {
        m_loc = fmaxf(m_loc, cst[t].m);
        mn_loc = fminf(mn_loc, cst[t].xmin);
    }
#pragma unroll
    for (int sft = 32; sft >= 1; sft >>= 1) {
        m_loc = fmaxf(m_loc, shxf(m_loc, sft));
        mn_loc = fminf(mn_loc, shxf(mn_loc, sft));
    }
    if ((tid & 63) == 0) {
        scx[tid >> 6] = m_loc;
        scq[tid >> 6] = mn_loc;
    }
    __syncthreads();
    float M = -INFINITY, XMIN = INFINITY;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        M = fmaxf(M, scx[i]);
        XMIN = fminf(XMIN, scq[i]);
    }
    __syncthreads();
    double z_loc = 0.0;
    for (int t = tid; t < nt; t += NT) {
        const ChunkStat cs = cst[t];
        if (cs.z != 0.0) z_loc += cs.z * exp_neg_tab((double)cs.m - (double)M, etab);
    }
    const double Z = wg_sum_f64<NT>(z_loc, scd);
    RowInfo info;
    info.kind = KIND_UNFILTERED;
    info.nK = P.V;
    info.T = 0;
    info.ZK = Z;
    info.m = M;
    info.xmin = XMIN;
    info.pad = 0;
    uint32_t idx;
    if (md.sm) {
        // the waves' race winners, compared exactly as inside the waves
        Race best;
        best.x = -INFINITY;
        best.qe = 1.0f;
        best.idx = NONE;
        best.lq = 0.0f;
        for (int t = tid; t < nt; t += NT) {
            const ChunkStat cs = cst[t];
            Race o;
            o.x = cs.rx;
            o.qe = cs.rqe;
            o.idx = cs.ridx;
            o.lq = 0.0f;
            if (race_ahead(o, best)) best = o;
        }
        idx = wg_race<NT>(best, scx, scq, sci).idx;
    } else {
        uint64_t am = 0;
        for (int t = tid; t < nt; t += NT)
            if (cst[t].ridx != NONE) {
                const uint64_t v = mkcomp(cst[t].rx, cst[t].ridx);
                am = v > am ? v : am;
            }
        am = wg_max_u64<NT>(am, sc64);
        idx = am ? cidx(am) : NONE;
        if (md.inv && am) info.m = cval(am);  // the row maximum, for the search
    }
    info.idx0 = idx;
    if (tid == 0) {
        P.out_idx[b] = (int64_t)idx;
        W.info[b] = info;
        // inverse-CDF draw over the whole row: the full-row search finds it
        if (md.inv && idx != NONE) W.fblist[atomicAdd(W.fbcnt, 1u)] = (uint32_t)b;
    }
}

__global__ __launch_bounds__(ROWS_THREADS) void k_rows(KParams P, KPlan L, KWork W) {
    __shared__ RowsShared S;
    // per-tile candidate offsets (L.nt PASS_WAVES + 1), then per-dense-tile
    // counts of the kept list (L.ntd + 1)
    extern __shared__ uint32_t toff[];
    constexpr int NT = ROWS_THREADS;
    const int tid = threadIdx.x;
    const int b = P.b0 + xcd_row(blockIdx.x, gridDim.x);
    // (read after the barriers that precede every use)
    if (tid < 64) S.etab[tid] = exp2_j64_tab[tid];
    const Mode md = row_mode(P, b);
    const bool filtered = md.tk || md.tp;
    const int nt = L.nt * PASS_WAVES;  // wave records (sub-slots) of the row
    const ChunkStat *cst = W.cstat + (int64_t)b * nt;

    // merged wave statistics (max, min, sum of exp), the records read in
    // parallel; rows with top-k need none of them
    auto merge_stats = [&](float &M, float &XMIN, double &Z) {
        float m_loc = -INFINITY, mn_loc = INFINITY;
        for (int t = tid; t < nt; t += NT) {
            m_loc = fmaxf(m_loc, cst[t].m);
            mn_loc = fminf(mn_loc, cst[t].xmin);
        }
#pragma unroll
        for (int sft = 32; sft >= 1; sft >>= 1) {
            m_loc = fmaxf(m_loc, shxf(m_loc, sft));
            mn_loc = fminf(mn_loc, shxf(mn_loc, sft));
        }
        if ((tid & 63) == 0) {
            S.scd[tid >> 6] = m_loc;
            S.scd[8 + (tid >> 6)] = mn_loc;
        }
        __syncthreads();
        M = -INFINITY;
        XMIN = INFINITY;
#pragma unroll
        for (int i = 0; i < NT / 64; ++i) {
            M = fmaxf(M, (float)S.scd[i]);
            XMIN = fminf(XMIN, (float)S.scd[8 + i]);
        }
        __syncthreads();
        double z_loc = 0.0;
        for (int t = tid; t < nt; t += NT) {
            const ChunkStat cs = cst[t];
            if (cs.z != 0.0) z_loc += cs.z * exp_neg_tab((double)cs.m - (double)M, S.etab);
        }
        Z = wg_sum_f64<NT>(z_loc, S.scd);
    };

    RowInfo info;
    info.kind = KIND_UNFILTERED;
    info.nK = P.V;
    info.T = 0;
    info.ZK = 0.0;
    info.m = -INFINITY;
    info.xmin = INFINITY;
    info.idx0 = NONE;
    info.pad = 0;

    if (!filtered) {
        merge_unfiltered<NT>(P, L, W, b, md, S.scd, S.sc64, S.scx, S.scq, S.sci, S.etab);
        return;
    }

    // ---- candidates of the row: the waves' sub-slots
    const uint32_t kk = md.tk ? (uint32_t)md.k : (uint32_t)min(P.guess, P.V);
    const float traw = W.rowthr[b];
    const uint64_t *rowc = W.cand + (int64_t)b * ROWCAP;
    uint32_t N;
    {
        // the sub-slot counts: exclusive prefix, overflows, and the entries
        // above the estimate's transform
        const int per = (nt + NT - 1) / NT;
        uint32_t loc = 0, chk = 0;  // chk: strict count + overflows << 16
        for (int i = 0; i < per; ++i) {
            const int t = tid * per + i;
            if (t < nt) {
                const uint32_t v = W.wcnt[b * nt + t];
                if (v == 0xffffffffu) {
                    chk += 1u << 16;
                } else {
                    loc += v & 0xffffu;
                    chk += v >> 16;
                }
            }
        }
        uint32_t tchk;
        (void)wg_excl_scan_u32<NT>(chk, S.sc, tchk);
        // The fast result is complete iff no wave overflowed and, unless the
        // estimate admitted everything, at least kk handed-over entries lie
        // above its transform (every element left out lies at or below it).
        // Otherwise the full-row search selects the row exactly.
        if ((tchk >> 16) != 0u || (traw > -INFINITY && (tchk & 0xffffu) < kk)) {
            info.kind = KIND_FALLBACK;
            info.idx0 = NONE;  // the row maximum is found by the search
            info.T = 0;
            if (tid == 0) {
                W.info[b] = info;
                W.fblist[atomicAdd(W.fbcnt, 1u)] = (uint32_t)b;
            }
            return;
        }
        uint32_t run = wg_excl_scan_u32<NT>(loc, S.sc, N);
        for (int i = 0; i < per; ++i) {
            const int t = tid * per + i;
            if (t < nt) {
                toff[t] = run;
                run += W.wcnt[b * nt + t] & 0xffffu;
            }
        }
        if (tid == 0) toff[nt] = N;
        __syncthreads();
    }
    const uint32_t tcap = (uint32_t)L.wcap;
    // entry e of the row's candidates
    auto gget = [&](uint32_t e) -> uint64_t {
        int lo = 0, hi = nt;  // toff[lo] <= e < toff[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (toff[mid] <= e) lo = mid;
            else hi = mid;
        }
        return rowc[(int64_t)lo * tcap + (e - toff[lo])];
    };

    // ---- the kk largest (exactly, under the composite order) into srt.  Up
    // to RCAP candidates are held in registers, RCAP / NT per thread, loaded
    // before the statistics are merged so that their latency overlaps it;
    // more (rare) are selected by passes over the slots themselves.
    uint32_t nsel = min(kk, N);
    const bool inreg = N <= (uint32_t)RCAP;
    // top-k keeping the ties at the k-th value: the selection grows to every
    // candidate with that value (the candidates hold all of them: every
    // element left out lies at or below the estimate's transform, below the
    // k-th value); a group too large for the list goes to the full-row
    // search with the k-th value as its floor
    const bool ties = md.tk && (P.flags & TOPK_TIES) != 0;
    // at most one wave's worth of candidates (the usual case for small k):
    // each is placed by counting the candidates above it instead of the
    // radix passes, and the selection, a prefix of the ordered candidates,
    // comes out in the row's order, so top-p below is a single scan
    const bool sorted = inreg && !ties && N <= (uint32_t)WAVE_TOPP;
    static_assert(WAVE_TOPP <= NT && WAVE_TOPP + 8 <= KMAX, "one candidate per thread, padded list");
    bool to_search = false;
    uint32_t kmin = 0;  // value key of the k-th largest (ties rows)
    constexpr int R = RCAP / NT;
    uint64_t v[R];
    uint32_t vm = 0;
    if (inreg) {
        // where candidate e lives, written slot by slot (a lookup per
        // candidate instead of a search over the slot offsets)
        for (int t = tid; t < nt; t += NT) {
            const uint32_t e0 = toff[t], e1 = toff[t + 1];
            for (uint32_t e = e0; e < e1; ++e) S.addr[e] = (uint32_t)t * tcap + (e - e0);
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t e = (uint32_t)(r * NT + tid);
            if (e < N) {
                v[r] = rowc[S.addr[e]];
                vm |= 1u << r;
            } else {
                v[r] = 0ull;
            }
        }
    }
    float M = -INFINITY, XMIN = INFINITY;
    double Z = 0.0;
    if (!md.tk) merge_stats(M, XMIN, Z);
    info.ZK = Z;
    info.m = M;
    info.xmin = XMIN;
    if (sorted) {
        // candidate e is v[0] of thread e; its place in the order is the
        // number of candidates above it (composites are distinct), counted
        // over broadcast reads of all of them, 8 per step (zero pads count
        // for nothing: no composite is 0)
        const uint32_t n8 = (N + 7u) & ~7u;
        if ((uint32_t)tid < N) S.srt[tid] = v[0];
        else if ((uint32_t)tid < n8) S.srt[tid] = 0ull;
        __syncthreads();
        uint32_t place = 0;
        if ((uint32_t)tid < N) {
            const uint64_t c = v[0];
            for (uint32_t j = 0; j < n8; j += 8) {
                uint64_t u[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) u[i] = S.srt[j + i];
#pragma unroll
                for (int i = 0; i < 8; ++i) place += u[i] > c ? 1u : 0u;
            }
        }
        __syncthreads();
        if ((uint32_t)tid < N && place < nsel) S.srt[place] = v[0];
    } else if (inreg) {
        uint32_t km = vm;
        if (N > kk) {
            uint64_t prefix, pmask;
            wg_radix_select<NT, R>(v, vm, kk, S.hist, S.sel, S.sc64, S.srt, KMAX, &S.sel[3],
                                   prefix, pmask);
            km = 0;
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (((vm >> r) & 1u) && (v[r] & pmask) >= prefix) km |= 1u << r;
        }
        if (ties) {
            uint32_t lo = ~0u;
#pragma unroll
            for (int r = 0; r < R; ++r)
                if ((km >> r) & 1u) lo = min(lo, (uint32_t)(v[r] >> 32));
            kmin = wg_min_u32<NT>(lo, S.sc);
            uint32_t km2 = 0;
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (((vm >> r) & 1u) && (uint32_t)(v[r] >> 32) >= kmin) km2 |= 1u << r;
            uint32_t n1;
            (void)wg_excl_scan_u32<NT>(__popc(km2), S.sc, n1);
            if (n1 > (uint32_t)KMAX) {
                to_search = true;
            } else {
                km = km2;
                nsel = n1;
            }
        }
        uint32_t tot;
        uint32_t off = wg_excl_scan_u32<NT>(__popc(km), S.sc, tot);
#pragma unroll
        for (int r = 0; r < R; ++r)
            if ((km >> r) & 1u) S.srt[off++] = v[r];
    } else {
        uint64_t prefix, pmask;
        radix_select_any<NT>(N, kk, gget, S.hist, S.sel, S.sc64, prefix, pmask);
        if (tid == 0) S.cnt = 0;
        __syncthreads();
        for (uint32_t e = tid; e < N; e += NT) {
            const uint64_t c = gget(e);
            if ((c & pmask) >= prefix) S.srt[atomicAdd(&S.cnt, 1u)] = c;
        }
        to_search = ties;  // (many candidates: rare) the full-row search does it
        if (ties) {
            __syncthreads();
            uint32_t lo = ~0u;
            for (uint32_t i = tid; i < nsel; i += NT) lo = min(lo, (uint32_t)(S.srt[i] >> 32));
            kmin = wg_min_u32<NT>(lo, S.sc);
        }
    }
    __syncthreads();

    // ---- the maximum and the softmax total, in double.  Thread tid owns
    // positions 4 tid .. 4 tid + 3 of srt.
    uint64_t v4[4];
    uint64_t mxv = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t p = 4 * tid + i;
        v4[i] = p < nsel ? S.srt[p] : 0ull;
        mxv = v4[i] > mxv ? v4[i] : mxv;
    }
    // a sampling row without top-p keeps the whole selection: q at its
    // entries is requested now, so that the gather overlaps what follows.
    // Every lane loads (id 0 past the selection): a load under a condition
    // would be waited for at once.
    const bool early_q = md.sm && !md.tp;
    float qv4[4];
    if (early_q) {
        const float *rowq = P.q + (int64_t)b * P.V;
#pragma unroll
        for (int i = 0; i < 4; ++i) qv4[i] = rowq[4 * tid + i < nsel ? cidx(v4[i]) : 0u];
    }
    // (an ordered selection starts with its maximum)
    const uint64_t top = sorted ? S.srt[0] : wg_max_u64<NT>(mxv, S.sc64);
    const float x0 = cval(top);
    if (to_search) {
        info.kind = KIND_FALLBACK;
        info.m = x0;
        info.idx0 = cidx(top);
        info.T = (uint64_t)kmin << 32;  // the floor: every value >= the k-th
        if (tid == 0) {
            W.info[b] = info;
            W.fblist[atomicAdd(W.fbcnt, 1u)] = (uint32_t)b;
        }
        return;
    }
    double loc = 0.0;
    double e4s[4];  // the masses of this thread's positions (0 past nsel)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        e4s[i] = 4 * tid + i < nsel ? exp_neg_tab((double)cval(v4[i]) - (double)x0, S.etab) : 0.0;
        loc += e4s[i];
    }
    const double tot_e = wg_sum_f64<NT>(loc, S.scd);
    double Zc;
    if (md.tk) Zc = tot_e;
    else Zc = (Z != 0.0) ? Z * exp_neg_tab((double)M - (double)x0, S.etab) : tot_e;

    // ---- top-p.  The kept set is the shortest prefix, in the order, whose
    // mass reaches p Zc.  Selections of at most WAVE_TOPP entries are sorted
    // and scanned by one wave; in larger ones short prefixes (the usual case)
    // are found by taking the maxima one at a time, longer ones by sorting
    // every candidate.
    uint32_t nK = nsel;
    bool settled = true;
    bool use_nuc = false;     // K is S.nuc[0..nK), else S.srt[0..nK)
    const bool small = nsel <= (uint32_t)WAVE_TOPP;  // all in wave 0 (positions 4 tid + i)
    const double pZ = md.tp ? (double)md.p * Zc : 0.0;
    double at = 0.0, below = 0.0;
    bool found = false;
    // ---- top-p without an inverse-CDF draw: K needs no order, only its
    // least element T*, so the selection is binned by value instead of
    // sorted.  256 bins from the top (bin 0 holds the largest values, -inf
    // the last bin) take the masses; the first bin whose running mass
    // reaches pZ holds T*; only its members are ranked, and K = { >= T* }
    // is written to srt in thread order.  The bins add masses (each <= 1,
    // the maximum's being 1) in fixed point, units of 2^-52, so that their
    // sums do not depend on the order of the atomics: the choice of bin is
    // then the same on every run, and off the double sums by at most nsel
    // 2^-52.
    const bool hist_cut = md.tp && !md.inv && !sorted;
    if (hist_cut) {
        double e4[4];
        uint32_t lo_key = ~0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t p = 4 * tid + i;
            const float x = cval(v4[i]);
            e4[i] = e4s[i];  // the softmax total's masses (0 past nsel)
            if (p < nsel && x > -INFINITY) lo_key = min(lo_key, (uint32_t)(v4[i] >> 32));
        }
        const uint32_t kmin_sel = wg_min_u32<NT>(lo_key, S.sc);
        const float span = kmin_sel == ~0u ? 0.0f : x0 - key2f(kmin_sel);
        const float scale = span > 0.0f && span < INFINITY ? 256.0f / span : 0.0f;
        uint64_t *hq = reinterpret_cast<uint64_t *>(S.addr);  // free by now
        uint64_t *bl = reinterpret_cast<uint64_t *>(S.addr) + 256;
        static_assert(sizeof(S.addr) >= (256 + KMAX) * sizeof(uint64_t), "bins and bucket");
        for (int i = tid; i < 256; i += NT) {
            hq[i] = 0ull;
            S.hist[i] = 0u;
        }
        __syncthreads();
        uint32_t bin4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x = cval(v4[i]);
            const float t = (x0 - x) * scale;
            bin4[i] = !(x > -INFINITY) ? 255u : (t >= 255.0f ? 255u : (uint32_t)t);
            if (4 * tid + i < nsel) {
                atomicAdd((unsigned long long *)&hq[bin4[i]],
                          (unsigned long long)(e4[i] * 0x1.0p52));
                atomicAdd(&S.hist[bin4[i]], 1u);
            }
        }
        __syncthreads();
        if (tid < 64) {
            // lane l sums bins 4 l .. 4 l + 3; the lane sums are scanned
            // with every lane active, and the first lane reaching pZ walks
            // its bins on top of the lanes before it
            double h[4];
            double ls = 0.0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                h[t] = (double)hq[4 * tid + t] * 0x1.0p-52;
                ls += h[t];
            }
            const double incl = wave_incl_scan_f64(ls, tid);
            const double excl = __shfl_up(incl, 1, 64);
            const uint64_t reach = __ballot(incl >= pZ);
            const int l = reach ? __builtin_ctzll(reach) : -1;
            if (tid == (l < 0 ? 0 : l)) {
                uint32_t pick = NONE;
                double acc = tid == 0 ? 0.0 : excl, pa = 0.0;
                if (l >= 0)
                    for (int t = 0; t < 4; ++t) {
                        if (h[t] > 0.0 && acc + h[t] >= pZ) {
                            pick = (uint32_t)(4 * tid + t);
                            pa = acc;
                            break;
                        }
                        acc += h[t];
                    }
                S.sel[0] = pick;
                S.fd[0] = pa;
            }
        }
        __syncthreads();
        const uint32_t bsel = S.sel[0];
        const double above_b = S.fd[0];
        if (bsel != NONE) {
            // the bucket's members, ranked by the number above each
            // (composites are distinct) into srt (the selection is in v4)
            if (tid == 0) S.cnt = 0u;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * tid + i < nsel && bin4[i] == bsel) bl[atomicAdd(&S.cnt, 1u)] = v4[i];
            __syncthreads();
            const uint32_t nb = S.cnt;
            for (uint32_t mi = tid; mi < nb; mi += NT) {
                const uint64_t c = bl[mi];
                uint32_t rank = 0;
                for (uint32_t j = 0; j < nb; ++j) rank += bl[j] > c ? 1u : 0u;
                S.srt[rank] = c;
            }
            __syncthreads();
            // running mass over the sorted bucket, 4 positions per thread
            double eb[4];
            double lb = 0.0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t p = 4 * tid + i;
                eb[i] = p < nb ? exp_neg_tab((double)cval(S.srt[p]) - (double)x0, S.etab) : 0.0;
                lb += eb[i];
            }
            double tb;
            double run = above_b + wg_excl_scan_f64<NT>(lb, S.scd, tb);
            uint32_t first = NONE;
            double a_ = 0.0, b_ = 0.0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t p = 4 * tid + i;
                run += eb[i];
                if (p < nb && first == NONE && run >= pZ) {
                    first = p;
                    a_ = run;
                    b_ = run - eb[i];
                }
                if (p + 1 == nb && first == NONE) {  // rounding: the whole bucket
                    a_ = run;
                    b_ = run - eb[i];
                }
            }
            const uint32_t mine = first;
            first = wg_min_u32<NT>(first, S.sc);
            const uint32_t fi = first == NONE ? nb - 1 : first;
            if ((first != NONE && mine == first) || (first == NONE && fi / 4 == (uint32_t)tid)) {
                S.fd[0] = a_;
                S.fd[1] = b_;
            }
            __syncthreads();
            const uint64_t tstar = S.srt[fi];
            found = true;
            at = S.fd[0];
            below = S.fd[1];
            __syncthreads();  // srt is rewritten below
            uint32_t kc = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) kc += (4 * tid + i < nsel && v4[i] >= tstar) ? 1u : 0u;
            uint32_t off = wg_excl_scan_u32<NT>(kc, S.sc, nK);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * tid + i < nsel && v4[i] >= tstar) S.srt[off++] = v4[i];
            __syncthreads();
        }
    }
    // ---- top-p, step 1: a short prefix (the usual case).  Small selections
    // take their 4 largest from one wave reduction; larger ones up to
    // NUC_STEPS maxima, one at a time, by the workgroup.
    if (md.tp && !hist_cut && !sorted) {
        if (small) {
            if (tid < 64) {
                uint64_t t4[4];
                wave_top4(v4, t4);  // v4 is 0 beyond nsel
                double cum = 0.0, prev = 0.0;
                uint32_t nfound = 0;
#pragma unroll
                for (int it = 0; it < WAVE_NUC; ++it) {
                    if (nfound || (uint32_t)it >= nsel) break;
                    prev = cum;
                    cum += exp_neg_tab((double)cval(t4[it]) - (double)x0, S.etab);
                    if (tid == 0) S.nuc[it] = t4[it];
                    if (cum >= pZ) nfound = it + 1;
                }
                if (tid == 0) {
                    S.sel[0] = nfound ? nfound - 1 : NONE;
                    S.fd[0] = cum;
                    S.fd[1] = prev;
                }
            }
            __syncthreads();
            if (S.sel[0] != NONE) {
                found = true;
                nK = S.sel[0] + 1;
                at = S.fd[0];
                below = S.fd[1];
            }
            __syncthreads();
        } else {
            uint32_t rem = 0;  // positions of this thread already taken
            double cum = 0.0;
            for (uint32_t it = 0; it < (uint32_t)NUC_STEPS && it < nsel; ++it) {
                uint64_t mx = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!((rem >> i) & 1u) && 4 * tid + i < nsel) mx = v4[i] > mx ? v4[i] : mx;
                mx = wg_max_u64<NT>(mx, S.sc64);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (v4[i] == mx && 4 * tid + i < nsel) rem |= 1u << i;
                const double em = exp_neg_tab((double)cval(mx) - (double)x0, S.etab);
                below = cum;
                cum += em;
                if (tid == 0) S.nuc[it] = mx;
                if (cum >= pZ) {
                    found = true;
                    at = cum;
                    nK = it + 1;
                    break;
                }
            }
        }
        use_nuc = found;
    }
    // ---- step 2: the selection in the row's order, when top-p needs more
    // than a short prefix, or for an inverse-CDF draw over the whole
    // selection.  Each wave sorts its 256 positions in registers; a small
    // selection is then wholly in wave 0, a larger one merges the four runs:
    // a key's place is its position in its run plus, in each other run, the
    // number of keys above it (a binary search; composite keys are distinct
    // and never 0, so 0 pads).  Then, for top-p, the shortest prefix whose
    // running mass (in double) reaches pZ.
    if (!hist_cut && (md.tp ? !found : (md.inv && nsel > 1))) {
        uint64_t w[4] = {v4[0], v4[1], v4[2], v4[3]};
        if (!sorted) wave_bitonic_desc256(w);
        if (small) {
            if (tid < 64) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if ((uint32_t)(4 * tid + i) < nsel) S.srt[4 * tid + i] = w[i];
            }
        } else {
            uint64_t *runs = reinterpret_cast<uint64_t *>(S.addr);  // free by now
#pragma unroll
            for (int i = 0; i < 4; ++i) runs[4 * tid + i] = w[i];
            __syncthreads();
            const int wv = tid >> 6;
#pragma unroll 1
            for (int i = 0; i < 4; ++i) {
                const uint64_t k = runs[4 * tid + i];
                if (k == 0ull) continue;
                uint32_t rank = (uint32_t)(4 * (tid & 63) + i);
#pragma unroll 1
                for (int o = 0; o < 4; ++o) {
                    if (o == wv) continue;
                    const uint64_t *r = runs + 256 * o;
                    uint32_t c = 0;  // keys above k: a prefix of the run
#pragma unroll
                    for (uint32_t step = 256; step >= 1; step >>= 1)
                        if (c + step <= 256u && r[c + step - 1] > k) c += step;
                    rank += c;
                }
                S.srt[rank] = k;
            }
        }
        __syncthreads();
        if (md.tp && small) {
            // wave 0: masses of its sorted registers, a shuffle scan, the
            // first position reaching pZ by ballot
            if (tid < 64) {
                double e[4];
                double l = 0.0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // an ordered selection has these masses already
                    e[i] = sorted ? e4s[i]
                                  : (4 * tid + i < nsel ? exp_neg_tab((double)cval(w[i]) - (double)x0, S.etab) : 0.0);
                    l += e[i];
                }
                const double inc = wave_incl_scan_f64(l, tid);
                double run = inc - l, a_ = 0.0, b_ = 0.0;
                uint32_t first = NONE;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t p = 4 * tid + i;
                    run += e[i];
                    if (p < nsel && first == NONE && run >= pZ) {
                        first = p;
                        a_ = run;
                        b_ = run - e[i];
                    }
                }
                const uint64_t hit = __ballot(first != NONE);
                if (hit == 0ull) {
                    if (tid == 0) S.sel[0] = NONE;
                } else if (tid == __ffsll((long long)hit) - 1) {
                    S.sel[0] = first;
                    S.fd[0] = a_;
                    S.fd[1] = b_;
                }
            }
            __syncthreads();
            if (S.sel[0] != NONE) {
                found = true;
                nK = S.sel[0] + 1;
                at = S.fd[0];
                below = S.fd[1];
            }
            __syncthreads();
        } else if (md.tp) {
            // workgroup: masses by position, an exclusive scan, the least
            // position reaching pZ
            double e[4];
            double l2 = 0.0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t p = 4 * tid + i;
                e[i] = p < nsel ? exp_neg_tab((double)cval(S.srt[p]) - (double)x0, S.etab) : 0.0;
                l2 += e[i];
            }
            double t2;
            const double before = wg_excl_scan_f64<NT>(l2, S.scd, t2);
            uint32_t first = NONE;
            double run = before, a_ = 0.0, b_ = 0.0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t p = 4 * tid + i;
                run += e[i];
                if (p < nsel && first == NONE && run >= pZ) {
                    first = p;
                    a_ = run;
                    b_ = run - e[i];
                }
            }
            const uint32_t mine = first;
            first = wg_min_u32<NT>(first, S.sc);
            if (first != NONE && mine == first) {
                S.fd[0] = a_;
                S.fd[1] = b_;
            }
            __syncthreads();
            if (first != NONE) {
                found = true;
                nK = first + 1;
                at = S.fd[0];
                below = S.fd[1];
            }
            __syncthreads();
        }
    }
    if (md.tp) {
        if (md.tk) {
            if (!found) nK = nsel;  // rounding: the whole top-k set
        } else if (!found) {
            // top-k guess (Ascend page, topP section): the guess does not
            // reach p; the full-row search decides
            settled = false;
        } else {
            // settled only when the cutoff lies inside the guess with a safe
            // margin on both sides
            const double hi_m = at - pZ;
            const double lo_m = (nK == 1) ? INFINITY : pZ - below;
            settled = (hi_m > GUESS_MARGIN * Zc && lo_m > GUESS_MARGIN * Zc) || md.p <= 0.0f;
        }
    }
    info.m = x0;
    info.idx0 = cidx(top);
    if (!settled) {
        info.kind = KIND_FALLBACK;
        if (tid == 0) {
            W.info[b] = info;
            W.fblist[atomicAdd(W.fbcnt, 1u)] = (uint32_t)b;
        }
        return;
    }
    __syncthreads();

    // ---- inverse-CDF draw over K, in the row's order (K is a prefix of
    // the sorted selection, or the short prefix in S.nuc)
    uint32_t inv_pos = 0;
    if (md.inv)
        inv_pos = inverse_cdf_pos<NT>(use_nuc ? S.nuc : S.srt, nK, x0, P.u[b], S.scd, S.sc, S.etab);

    // ---- exponential race over K (or greedy), and the kept list
    const uint64_t *kp = use_nuc ? S.nuc : S.srt;
    uint32_t idx = cidx(top);
    if (md.inv) idx = cidx(kp[inv_pos]);
    double zk = 0.0;
    double rbest = -1.0;
    uint32_t ibest = NONE;
    uint64_t *kl = W.klist + (int64_t)b * KMAX;
    constexpr int KR = KMAX / NT;
    float qv[KR];
    if (md.sm && !early_q) {
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            const uint32_t p = (uint32_t)(r * NT + tid);
            const uint32_t id = p < nK ? cidx(kp[p]) : 0u;  // every lane loads
            qv[r] = P.q[(int64_t)b * P.V + id];
        }
    }
    if (early_q) {
        // K is the whole selection: each thread races its own entries
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * tid + i < nsel) {
                const uint32_t id = cidx(v4[i]);
                const double ei = e4s[i];
                const double rr = race_ratio(cval(v4[i]), ei, (double)qv4[i] + (double)P.eps);
                if (rr > rbest || (rr == rbest && id < ibest)) {
                    rbest = rr;
                    ibest = id;
                }
            }
    }
    // for the dense outputs, the kept list goes out grouped by tile (any
    // order within a tile), so that each dense-writer workgroup reads only
    // its own entries; toff (no longer needed for the candidates) counts them
    // per tile
    const int ntile = L.ntd;
    const bool group = P.out_probs != nullptr || P.out_logits != nullptr;
    if (group) {
        for (int i = tid; i <= ntile; i += NT) toff[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            const uint32_t p = (uint32_t)(r * NT + tid);
            if (p < nK) atomicAdd(&toff[dense_tile(cidx(kp[p]), (uint32_t)ntile)], 1u);
        }
        __syncthreads();
        const int per = (ntile + NT - 1) / NT;
        uint32_t lc = 0;
        for (int i = 0; i < per; ++i) {
            const int t = tid * per + i;
            if (t < ntile) lc += toff[t];
        }
        uint32_t tot2;
        uint32_t run = wg_excl_scan_u32<NT>(lc, S.sc, tot2);
        for (int i = 0; i < per; ++i) {
            const int t = tid * per + i;
            if (t < ntile) {
                const uint32_t c = toff[t];
                toff[t] = run;
                W.ktoff[(int64_t)b * (ntile + 1) + t] = run;
                run += c;
            }
        }
        if (tid == 0) W.ktoff[(int64_t)b * (ntile + 1) + ntile] = nK;
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < KR; ++r) {
        const uint32_t p = (uint32_t)(r * NT + tid);
        if (p < nK) {
            const uint64_t v = kp[p];
            const uint32_t id = cidx(v);
            const double ei = exp_neg_tab((double)cval(v) - (double)x0, S.etab);
            zk += ei;
            if (md.sm && !early_q) {
                const double rr = race_ratio(cval(v), ei, (double)qv[r] + (double)P.eps);
                if (rr > rbest || (rr == rbest && id < ibest)) {
                    rbest = rr;
                    ibest = id;
                }
            }
            if (group) kl[atomicAdd(&toff[dense_tile(id, (uint32_t)ntile)], 1u)] = v;
        }
    }
    if (md.sm) idx = wg_best_ratio<NT>(rbest, ibest, S.scd, S.sci);
    zk = wg_sum_f64<NT>(zk, S.scd);
    info.kind = KIND_LIST;
    info.nK = (int32_t)nK;
    info.ZK = zk;
    if (tid == 0) {
        P.out_idx[b] = (int64_t)idx;
        W.info[b] = info;
    }
}

// ================================================================== k_fallback

struct FallbackShared {
    double hm[K3_BINS];
    uint32_t hc[K3_BINS];
    uint32_t hlo[K3_BINS];
    uint32_t hhi[K3_BINS];
    uint64_t coll[K3_COLLECT];
    uint64_t rk[K3_BINS];  // first level: the best race key of each bin (race_key)
    double etab[64];       // 2^(j/64) for exp_neg_tab
    uint32_t bm[K3_SEG / 32];
    // refinement levels: level 0 bins by value, later levels by key
    float lv_lo, lv_scale;
    uint32_t lv_bin[8];
    uint32_t lv_klo[8];
    uint32_t lv_sh[8];
    uint32_t sc[16];
    uint64_t sc64[16];
    double scd[16];
    float scx[16], scq[16];
    uint32_t sci[16];
    uint32_t counter;
    uint32_t found[4];
    double fd[4];
    double lane_sum[64];
};

__device__ __forceinline__ uint32_t bin_value(float x, float lo, float scale) {
    // below lo (and NaN) -> 0, from K3_BINS - 1 up -> K3_BINS - 1, without
    // branches (fmaxf of NaN and 0 is 0)
    const float t = fminf(fmaxf((x - lo) * scale, 0.0f), (float)(K3_BINS - 1));
    return (uint32_t)t;
}
// Key bins of a refinement level: keys from klo on, 2^sh keys per bin (sh
// makes the parent bucket's key range fit the K3_BINS bins).
__device__ __forceinline__ uint32_t bin_key(uint32_t key, uint32_t klo, uint32_t sh) {
    const uint32_t bi = (key - klo) >> sh;
    return bi < (uint32_t)K3_BINS ? bi : (uint32_t)(K3_BINS - 1);
}
// Smallest sh with (span - 1) >> sh < K3_BINS, for a key range of `span` keys.
__device__ __forceinline__ uint32_t bin_shift(uint64_t span) {
    const int bits = span > 1 ? 64 - __clzll((long long)(span - 1)) : 0;
    constexpr int BB = 11;  // log2(K3_BINS)
    static_assert((1 << BB) == K3_BINS, "K3_BINS is a power of two");
    return bits > BB ? (uint32_t)(bits - BB) : 0u;
}

// A race candidate as one 64-bit key that atomicMax can keep per bin: the
// ratio e / den in double (0 for a -inf logit, +inf over a zero
// denominator; a non-negative double orders like its bit pattern) cut to its
// top 43 bits (relative steps of 2^-31), then ~id in the low 21 bits, so
// that of two ratios that agree to that precision the smaller id wins.  Ids
// are below SAMPLER_VOCAB_MAX = 2^21.  The keys only choose each bin's
// candidate: the winner is decided afresh by exact ratios.
constexpr int RK_ID_BITS = 21;
static_assert((1 << RK_ID_BITS) >= SAMPLER_VOCAB_MAX, "ids fit the key's low bits");
__device__ __forceinline__ uint64_t race_key(float x, double e, double den, uint32_t j) {
    // e times the reciprocal of den (a hardware estimate and one Newton
    // step, good to a few units in the last place: far inside the key's
    // 2^-31 cut), not a division
    double y = __builtin_amdgcn_rcp(den);
    y = fma(fma(-den, y, 1.0), y, y);
    const double r = !(x > -INFINITY) ? 0.0 : (den == 0.0 ? (double)INFINITY : e * y);
    const uint64_t hi = (uint64_t)__double_as_longlong(r) >> RK_ID_BITS;
    return (hi << RK_ID_BITS) | (uint64_t)(~j & ((1u << RK_ID_BITS) - 1u));
}
__device__ __forceinline__ uint32_t race_key_id(uint64_t k) {
    return ~(uint32_t)k & ((1u << RK_ID_BITS) - 1u);
}

// Boundary bucket of a mass histogram: walking the bins from the top, the
// bin where the running mass first reaches `need`.  Writes found[0] = bin,
// fd[0] = the mass of the bins above it, the running sum that the choice was
// made with, so exactly one bin is chosen whatever the rounding.  Wave 0
// sums 32 bins per lane and scans the lane sums; the first lane whose
// inclusive sum reaches `need` scans its 32 bins on top of the lanes before
// it, and the first bin of mass > 0 reaching `need` is the bucket.  When
// rounding leaves no such bin in that lane, lane 0 walks the lane sums and
// bins one by one instead, and if `need` lies beyond the total it takes the
// lowest non-empty bin.
__device__ void find_bucket(const double *hm, const uint32_t *hc, double need, double *lane_sum,
                            uint32_t *found, double *fd) {
    constexpr int PER = K3_BINS / 64;
    static_assert(PER <= 64, "one lane per bin of a lane's share");
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        double s = 0.0;
        for (int t = 0; t < PER; ++t) s += hm[K3_BINS - 1 - lane * PER - t];
        lane_sum[lane] = s;
        const double incl = wave_incl_scan_f64(s, lane);
        const double excl = __shfl_up(incl, 1, 64);
        const uint64_t reach = __ballot(incl >= need);
        bool done = false;
        if (reach) {
            const int l = __builtin_ctzll(reach);
            // shuffles run with every lane active (a lane outside the
            // active set would read as 0), their results selected after
            const double excl_l = __shfl(excl, l, 64);
            const double acc0 = l == 0 ? 0.0 : excl_l;
            const int bin = K3_BINS - 1 - l * PER - lane;
            const double mb = lane < PER ? hm[bin] : 0.0;
            const double bi = wave_incl_scan_f64(mb, lane);
            const double bi_up = __shfl_up(bi, 1, 64);
            const double be = lane == 0 ? 0.0 : bi_up;
            const double acc = acc0 + be;
            const uint64_t hit = __ballot(lane < PER && mb > 0.0 && acc + mb >= need);
            if (hit) {
                const int t = __builtin_ctzll(hit);
                if (lane == t) {
                    found[0] = (uint32_t)bin;
                    fd[0] = acc;
                }
                done = true;
            }
        }
        if (lane == 0) found[3] = done ? 1u : 0u;
    }
    __syncthreads();
    if (threadIdx.x == 0 && found[3] == 0u) {
        double acc = 0.0;
        int l = 0;
        for (; l < 63; ++l) {
            if (acc + lane_sum[l] >= need) break;
            acc += lane_sum[l];
        }
        uint32_t pick = NONE, last_nonempty = NONE;
        double pick_above = 0.0, last_above = 0.0;
        for (int ll = l; ll < 64 && pick == NONE; ++ll) {
            for (int t = 0; t < PER; ++t) {
                const int bin = K3_BINS - 1 - ll * PER - t;
                const double mbin = hm[bin];
                if (hc[bin] > 0) {
                    last_nonempty = (uint32_t)bin;
                    last_above = acc;
                }
                if (mbin > 0.0 && acc + mbin >= need) {
                    pick = (uint32_t)bin;
                    pick_above = acc;
                    break;
                }
                acc += mbin;
            }
        }
        if (pick == NONE) {
            pick = (last_nonempty == NONE) ? 0u : last_nonempty;
            pick_above = last_above;
        }
        found[0] = pick;
        fd[0] = pick_above;
    }
    __syncthreads();
}

// Is x (key k) inside the selected bucket of every level < nlev?
__device__ __forceinline__ bool in_play(const FallbackShared &S, float x, uint32_t k, int nlev) {
    if (nlev == 0) return true;
    if (bin_value(x, S.lv_lo, S.lv_scale) != S.lv_bin[0]) return false;
    for (int l = 1; l < nlev; ++l)
        if (bin_key(k, S.lv_klo[l], S.lv_sh[l]) != S.lv_bin[l]) return false;
    return true;
}

// Visit every element (x transformed, id j) of elements [c0, c1) of row b;
// f(x, j).  c0 is a multiple of 4.  Groups of 4 per thread, the next group
// requested before the current one is visited, so that each thread keeps a
// load in flight while its visitors run.
template <int DT, bool AL, bool XF, class F>
__device__ __forceinline__ void range_pass(const KParams &P, int b, int c0, int c1, uint32_t *bm,
                                           F &&f) {
    const void *rowp = row_ptr(P, DT, b);
    for (int s0 = c0; s0 < c1; s0 += K3_SEG) {
        const int s1 = min(s0 + K3_SEG, c1);
        if (P.pen) build_bitmap<K3_THREADS>(bm, s0, s1 - s0, P, b);
        int j = s0 + (int)threadIdx.x * 4;
        Raw4<DT> rx;
        if (j < s1) load4<DT, AL>(rowp, j, s1 - j >= 4 ? 4 : s1 - j, rx);
        for (; j < s1; j += K3_THREADS * 4) {
            const int nv = s1 - j >= 4 ? 4 : s1 - j;
            float x[4];
            unpack4<DT>(rx, x);
            const int jn = j + K3_THREADS * 4;
            if (jn < s1) load4<DT, AL>(rowp, jn, s1 - jn >= 4 ? 4 : s1 - jn, rx);
            uint32_t bits = 0;
            if (P.pen) {
                const int r = j - s0;
                bits = (bm[r >> 5] >> (r & 31)) & 0xfu;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < nv) f(xform<XF>(x[i], (bits >> i) & 1u, P), (uint32_t)(j + i));
        }
    }
    __syncthreads();
}

template <int DT, bool AL, bool XF, class F>
__device__ __forceinline__ void row_pass(const KParams &P, int b, uint32_t *bm, F &&f) {
    range_pass<DT, AL, XF>(P, b, 0, P.V, bm, f);
}

// range_pass with the row's q as well, f(x, q, j), in groups of 4: the 4
// logits and the 4 q of a group are requested as vectors one group ahead of
// the visitors, so a visitor that needs q only for some elements does not
// wait for each load in turn (and 4-wide groups keep the register count
// down).
template <int DT, bool AL, bool XF, class F>
__device__ __forceinline__ void range_pass_q(const KParams &P, int b, int c0, int c1, uint32_t *bm,
                                             const float *rowq, F &&f) {
    const void *rowp = row_ptr(P, DT, b);
    for (int s0 = c0; s0 < c1; s0 += K3_SEG) {
        const int s1 = min(s0 + K3_SEG, c1);
        if (P.pen) build_bitmap<K3_THREADS>(bm, s0, s1 - s0, P, b);
        // one group in flight ahead of the one being visited
        int j = s0 + (int)threadIdx.x * 4;
        Raw4<DT> rx;
        Raw4<0> rq;
        if (j < s1) {
            const int nv0 = s1 - j >= 4 ? 4 : s1 - j;
            load4<DT, AL>(rowp, j, nv0, rx);
            load4<0, AL>(rowq, j, nv0, rq);
        }
        for (; j < s1; j += K3_THREADS * 4) {
            const int nv = s1 - j >= 4 ? 4 : s1 - j;
            float x[4], qx[4];
            unpack4<DT>(rx, x);
            unpack4<0>(rq, qx);
            const int jn = j + K3_THREADS * 4;
            if (jn < s1) {
                const int nvn = s1 - jn >= 4 ? 4 : s1 - jn;
                load4<DT, AL>(rowp, jn, nvn, rx);
                load4<0, AL>(rowq, jn, nvn, rq);
            }
            uint32_t bits = 0;
            if (P.pen) {
                const int r = j - s0;
                bits = (bm[r >> 5] >> (r & 31)) & 0xfu;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < nv) f(xform<XF>(x[i], (bits >> i) & 1u, P), qx[i], (uint32_t)(j + i));
        }
    }
    __syncthreads();
}

template <int DT, bool AL, bool XF, class F>
__device__ __forceinline__ void row_pass_q(const KParams &P, int b, uint32_t *bm, const float *rowq,
                                           F &&f) {
    range_pass_q<DT, AL, XF>(P, b, 0, P.V, bm, rowq, f);
}

// Visit the elements of [c0, c1) of row b (c0 a multiple of 4) whose
// transformed key lies in [klo, khi]; f(x, j).  A pass of one workgroup over
// a row is bound by its instruction count and by the loads each thread
// keeps in flight, so the key test comes first and whole chunks of KS_D
// groups of 4 per thread are requested at once (unconditional loads); the
// tail of each bitmap segment goes one group per thread.
constexpr int KS_D = 4;
template <int DT, bool AL, bool XF, class F>
__device__ __forceinline__ void key_scan(const KParams &P, int b, int c0, int c1, uint32_t klo,
                                         uint32_t khi, uint32_t *bm, F &&f) {
    constexpr int STEP = K3_THREADS * 4;
    constexpr int CHUNK = STEP * KS_D;
    const void *rowp = row_ptr(P, DT, b);
    const int t4 = (int)threadIdx.x * 4;
    auto visit4 = [&](const Raw4<DT> &r, int j, int nv, int s0) {
        float x[4];
        unpack4<DT>(r, x);
        uint32_t bits = 0;
        if (P.pen) {
            const int rr = j - s0;
            bits = (bm[rr >> 5] >> (rr & 31)) & 0xfu;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (i < nv) {
                const float y = xform<XF>(x[i], (bits >> i) & 1u, P);
                const uint32_t k = f2key(y);
                if (k >= klo && k <= khi) f(y, (uint32_t)(j + i));
            }
    };
    for (int s0 = c0; s0 < c1; s0 += K3_SEG) {
        const int s1 = min(s0 + K3_SEG, c1);
        if (P.pen) build_bitmap<K3_THREADS>(bm, s0, s1 - s0, P, b);
        int base = s0;
        for (; base + CHUNK <= s1; base += CHUNK) {
            Raw4<DT> r[KS_D];
#pragma unroll
            for (int d = 0; d < KS_D; ++d) load4<DT, AL>(rowp, base + d * STEP + t4, 4, r[d]);
#pragma unroll
            for (int d = 0; d < KS_D; ++d) visit4(r[d], base + d * STEP + t4, 4, s0);
        }
        for (int j = base + t4; j < s1; j += STEP) {
            Raw4<DT> r;
            const int nv = nv4(j, s1);
            load4<DT, AL>(rowp, j, nv, r);
            visit4(r, j, nv, s0);
        }
    }
    __syncthreads();
}

// Bin function of the first histogram level of a row's search: bins over the
// values that take part, from about the row minimum (or the floor's value)
// to the maximum m, at most 128 below it; smaller values (whose mass is
// below 1e-55 of the maximum's) fall in bin 0.
__device__ __forceinline__ void level0_bins(float m, float rowlo, uint64_t cfloor, float &lo,
                                            float &scale) {
    lo = m - 128.0f;
    if (rowlo <= m) lo = fmaxf(lo, rowlo);
    if (cfloor != 0) lo = fmaxf(lo, key2f((uint32_t)(cfloor >> 32)));
    const float w = m - lo;
    scale = w > 0.0f ? (float)K3_BINS / w : 1.0f;
    if (!(scale < INFINITY)) scale = 1.0f;  // a one-value range
}

// Keys of first-level bin fb's value range, half a bin wider on each side
// than its edges (rounding in bin_value moves an edge by far less), and 64
// keys more (adjacent floats have adjacent keys) for bins narrower than a
// unit in the last place of their values; bin 0 also holds everything below
// lo (-inf included), the last bin everything up to the maximum m.
// Membership is decided by the bin itself; the range only has to hold every
// member.
__device__ __forceinline__ void level0_keys(uint32_t fb, float lo, float scale, float m,
                                            uint32_t &klo, uint32_t &khi) {
    const float w = 1.0f / scale;
    klo = fb == 0 ? 0u : f2key(lo + ((float)fb - 0.5f) * w);
    khi = fb == (uint32_t)(K3_BINS - 1) ? f2key(m) : f2key(fminf(lo + ((float)fb + 1.5f) * w, m));
    if (khi < klo) khi = klo;
    klo = klo > 64u ? klo - 64u : 0u;
    khi = khi < 0xffffffffu - 64u ? khi + 64u : 0xffffffffu;
}

// A tile's partial first level in the workspace: masses, race keys, counts
// of the K3_BINS bins, its total mass, then per chunk of FB_CHUNK_BINS bins
// (chunk c: bins K3_BINS - 1 - c FB_CHUNK_BINS down, the order in which the
// bucket search sums them) the chunk's mass and its largest race key.
constexpr int FB_CHUNK_BINS = K3_BINS / FB_CHUNKS;
static_assert(FB_CHUNKS == 64 && FB_CHUNK_BINS <= 64, "one lane per chunk, one lane per bin");
struct FbPart {
    double *hm;
    uint64_t *rk;
    uint32_t *hc;
    double *z;
    double *csum;
    uint64_t *crk;
};
// The bucket members the tiles of a row list for its last tile: in the
// row's first part slot, once the parts are merged.
static_assert(FB_PART_BYTES >= (size_t)K3_COLLECT * 8, "member list fits a part slot");
__device__ __forceinline__ uint64_t *fb_members(char *base, uint32_t slot0) {
    return reinterpret_cast<uint64_t *>(base + (size_t)slot0 * FB_PART_BYTES);
}
__device__ __forceinline__ FbPart fb_part(char *base, uint32_t slot) {
    char *p = base + (size_t)slot * FB_PART_BYTES;
    FbPart f;
    f.hm = (double *)p;
    f.rk = (uint64_t *)(p + (size_t)K3_BINS * 8);
    f.hc = (uint32_t *)(p + (size_t)K3_BINS * 16);
    f.z = (double *)(p + (size_t)K3_BINS * 20);
    f.csum = (double *)(p + FB_PART_CHUNKS);
    f.crk = (uint64_t *)(p + FB_PART_CHUNKS + (size_t)FB_CHUNKS * 8);
    return f;
}


template <int DT, bool AL, bool XF>
__global__ __launch_bounds__(K3_THREADS) void k_fallback(KParams P, KPlan L, KWork W) {
    __shared__ FallbackShared S;
    const int tid = threadIdx.x;
    if (tid < 64) S.etab[tid] = exp2_j64_tab[tid];
    __syncthreads();
    // The rows the merge queued, spread over the workgroups.  While the
    // queue is short (T > 1), the first histogram level of the cut's search
    // of a row is split into T tiles, one workgroup each: each writes its
    // partial histogram, and the last to arrive merges them (in tile order)
    // and carries on with the row alone.
    const uint32_t nq = *W.fbcnt;
    const FbTiling ft = fb_tiling(nq, gridDim.x, P.V);
    const uint32_t ntiles = (uint32_t)ft.T;
    for (uint32_t it = blockIdx.x; it < nq * ntiles; it += gridDim.x) {
    const uint32_t qi = it / ntiles, tile = it % ntiles;
    const int b = (int)W.fblist[qi];
    RowInfo info = W.info[b];
    const Mode md = row_mode(P, b);
    // queued only for an inverse-CDF draw over the whole row
    const bool whole = info.kind == KIND_UNFILTERED;
    // tiles take the first level of the first search when that search is
    // the cut's (or the whole-row draw's) at a positive level and the row's
    // maximum is known
    const bool tiled = ntiles > 1 && info.idx0 != NONE &&
                       (whole ? P.u[b] > 0.0f
                              : (md.tp && md.p > 0.0f && !(md.tk && info.T == 0)));
    if (!tiled && tile != 0) continue;
    if (info.idx0 == NONE) {
        // a row the merge found incomplete: its maximum (the first element of
        // the order) from one pass over the row
        uint64_t mx = 0;
        row_pass<DT, AL, XF>(P, b, S.bm, [&](float x, uint32_t j) {
            const uint64_t c = mkcomp(x, j);
            mx = c > mx ? c : mx;
        });
        mx = wg_max_u64<K3_THREADS>(mx, S.sc64);
        info.m = cval(mx);
        info.idx0 = cidx(mx);
    }
    const double m = (double)info.m;
    uint64_t cfloor = info.T;  // only composites >= cfloor take part (0: all)
    // low end of the first histogram level: the smallest value of the row's
    // estimate sample (rows with top-k / top-p; elements below it share bin
    // 0, which later levels refine like any other bin)
    const float rowlo = (md.tk || md.tp) ? W.rowlo[b] : INFINITY;

    // The least element T* (a composite) of the row's order at which the
    // weight summed from the top reaches the target -- tval times the total
    // weight (found on the first pass) when frac, else tval itself -- and
    // ZKo, the weight through T*.  The weight of an element is exp(x - m), or
    // 1 when count (then -inf values count too).
    // With rk_on (the cut of a sampling row) the first level also keeps each
    // bin's best race key, and when the search ends at that level (its
    // boundary bucket collected) rk_top is the best key of the bins above the
    // boundary and rk_fi the last kept position of the sorted bucket: the race
    // over K then needs no pass of its own.
    bool rk_done = false;
    uint64_t rk_top = 0;
    uint32_t rk_fi = 0;
    const float *rowq = md.sm ? P.q + (int64_t)b * P.V : nullptr;

    // The tiles of a tiled row: this workgroup's part of the first level of
    // the first search (weights exp(x - m), race keys for a sampling row's
    // cut), written to its slot it = qi * T + tile.  The last tile to arrive
    // merges the T parts into S (masses, counts and totals summed in tile
    // order, keys by maximum) for that search to use.
    bool pre0 = false;
    double pre_z = 0.0;
    if (tiled) {
        const bool rkt = md.sm && !whole;
        float lo, scale;
        level0_bins(info.m, rowlo, cfloor, lo, scale);
        for (int i = tid; i < K3_BINS; i += K3_THREADS) {
            S.hm[i] = 0.0;
            S.hc[i] = 0u;
            if (rkt) S.rk[i] = 0ull;
        }
        __syncthreads();
        const int c0 = (int)tile * ft.TL, c1 = min(c0 + ft.TL, P.V);
        double zt = 0.0;
        auto visit = [&](float x, uint32_t j, float qj) {
            if (!(x > -INFINITY) || mkcomp(x, j) < cfloor) return;
            const double e = exp_neg_tab((double)x - m, S.etab);
            zt += e;
            const uint32_t bi = bin_value(x, lo, scale);
            atomicAdd(&S.hm[bi], e);
            atomicAdd(&S.hc[bi], 1u);
            if (rkt) atomicMax(&S.rk[bi], race_key(x, e, (double)qj + (double)P.eps, j));
        };
        if (rkt)
            range_pass_q<DT, AL, XF>(P, b, c0, c1, S.bm, rowq,
                                     [&](float x, float qj, uint32_t j) { visit(x, j, qj); });
        else
            range_pass<DT, AL, XF>(P, b, c0, c1, S.bm,
                                   [&](float x, uint32_t j) { visit(x, j, 0.0f); });
        const double zsum = wg_sum_f64<K3_THREADS>(zt, S.scd);
        const FbPart mine = fb_part(W.fbpart, it);
        // the part goes out by device-scope stores (written through to the
        // level every workgroup reads), so that the release below has little
        // left to write back
        for (int i = tid; i < K3_BINS; i += K3_THREADS) {
            __hip_atomic_store(&mine.hm[i], S.hm[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&mine.hc[i], S.hc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (rkt)
                __hip_atomic_store(&mine.rk[i], S.rk[i], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        if (tid == 0) __hip_atomic_store(mine.z, zsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the chunk summaries: 32 lanes per chunk, summed by shuffles
        static_assert(FB_CHUNK_BINS == 32, "a chunk is half a wave");
        for (int c0 = 0; c0 < FB_CHUNKS; c0 += K3_THREADS / FB_CHUNK_BINS) {
            const int c = c0 + tid / FB_CHUNK_BINS;
            const int i = K3_BINS - 1 - c * FB_CHUNK_BINS - (tid % FB_CHUNK_BINS);
            double cs = S.hm[i];
            uint64_t ck = rkt ? S.rk[i] : 0ull;
#pragma unroll
            for (int sft = FB_CHUNK_BINS / 2; sft >= 1; sft >>= 1) {
                cs += shxd(cs, sft);
                const uint64_t o = shx64(ck, sft);
                ck = o > ck ? o : ck;
            }
            if (tid % FB_CHUNK_BINS == 0) {
                __hip_atomic_store(&mine.csum[c], cs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&mine.crk[c], ck, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        // One thread counts the arrival: its release publishes the whole part,
        // and the last tile's acquire makes every part visible to the
        // workgroup past the next barrier.  Each wave first waits for its own
        // stores to complete (requests of different waves to different
        // memory channels are not ordered by the barrier), so that they
        // precede the release; only that thread touches the device-wide
        // cache state.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        uint32_t *sy = W.fbsync + (size_t)qi * FB_SYNC_WORDS;
        if (tid == 0) {
            const uint32_t old =
                __hip_atomic_fetch_add(&sy[0], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            if (old == ntiles - 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            S.found[2] = old;
        }
        __syncthreads();
        if (S.found[2] != ntiles - 1) {
            // A later tile finishes the row.  This one waits, for at most
            // FB_POLLS polls, for the first-level bucket the last tile
            // publishes, collects the bucket's members in its own range and
            // lists them in the row's first part slot (the parts are merged
            // by then).  Giving up only leaves the collection to the last
            // tile, which then reads the whole row itself.
            if (tid == 0) {
                uint32_t v = 0u;
                for (int it = 0; it < FB_POLLS; ++it) {
                    v = __hip_atomic_load(&sy[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (v != 0u) break;
                    __builtin_amdgcn_s_sleep(8);
                }
                S.found[3] = v;
            }
            __syncthreads();
            const uint32_t pub = S.found[3];
            if (pub == 0u || pub == FB_NO_BUCKET) continue;
            const uint32_t fbp = pub - 1u;
            uint32_t kl, kh;
            level0_keys(fbp, lo, scale, info.m, kl, kh);
            if (tid == 0) S.counter = 0u;
            __syncthreads();
            key_scan<DT, AL, XF>(P, b, c0, c1, kl, kh, S.bm, [&](float x, uint32_t j) {
                if (!(x > -INFINITY) || mkcomp(x, j) < cfloor) return;
                if (bin_value(x, lo, scale) != fbp) return;
                const uint32_t pos = atomicAdd(&S.counter, 1u);
                if (pos < (uint32_t)K3_COLLECT) S.coll[pos] = mkcomp(x, j);
            });
            const uint32_t nc = min(S.counter, (uint32_t)K3_COLLECT);
            if (tid == 0)
                S.found[1] = __hip_atomic_fetch_add(&sy[3], nc, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            const uint32_t base = S.found[1];
            uint64_t *mem = fb_members(W.fbpart, qi * ntiles);
            for (uint32_t i = tid; i < nc; i += K3_THREADS)
                if (base + i < (uint32_t)K3_COLLECT) mem[base + i] = S.coll[i];
            // every wave's list stores complete before the release (as above)
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid == 0)
                __hip_atomic_fetch_add(&sy[2], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            continue;
        }
        // the tiles' totals, read at once and summed in tile order
        static_assert(FB_TILES_MAX <= 16, "one scratch entry per tile");
        if (tid < (int)ntiles) S.scd[tid] = *fb_part(W.fbpart, qi * ntiles + tid).z;
        __syncthreads();
        for (uint32_t t = 0; t < ntiles; ++t) pre_z += S.scd[t];
        __syncthreads();
        pre0 = true;
    }

    // The tiles' parts merged bin by bin, in tile order, into the first
    // level's histogram in S (what a one-workgroup first level would hold).
    auto merge_parts = [&](bool rkt) {
        const uint32_t slot0 = qi * ntiles;
        // each thread merges its K3_BINS / K3_THREADS bins, the loads of four
        // tiles requested together; the sums still run in tile order
        constexpr int BPT = K3_BINS / K3_THREADS;
        static_assert(BPT * K3_THREADS == K3_BINS, "bins per thread");
        double hm[BPT];
        uint32_t hc[BPT];
        uint64_t rk[BPT];
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
            hm[u] = 0.0;
            hc[u] = 0u;
            rk[u] = 0ull;
        }
        for (uint32_t t0 = 0; t0 < ntiles; t0 += 4) {
            double a[4][BPT];
            uint32_t c[4][BPT];
            uint64_t k[4][BPT];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const FbPart pt = fb_part(W.fbpart, slot0 + min(t0 + v, ntiles - 1));
#pragma unroll
                for (int u = 0; u < BPT; ++u) {
                    const int i = tid + u * K3_THREADS;
                    a[v][u] = pt.hm[i];
                    c[v][u] = pt.hc[i];
                    k[v][u] = pt.rk[i];  // read whether or not written: kept only with rkt
                }
            }
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (t0 + v < ntiles) {
#pragma unroll
                    for (int u = 0; u < BPT; ++u) {
                        hm[u] += a[v][u];
                        hc[u] += c[v][u];
                        rk[u] = k[v][u] > rk[u] ? k[v][u] : rk[u];
                    }
                }
        }
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
            const int i = tid + u * K3_THREADS;
            S.hm[i] = hm[u];
            S.hc[i] = hc[u];
            if (rkt) S.rk[i] = rk[u];
            S.hlo[i] = NONE;
            S.hhi[i] = 0u;
        }
        __syncthreads();
    };

    // The boundary bucket of the merged first level from the tiles' chunk
    // summaries and the bins of one chunk only: wave 0 merges the chunk masses
    // (tile order), takes the first chunk whose running sum reaches need,
    // merges that chunk's bins and takes the first bin of mass > 0 reaching
    // need, as find_bucket would on the merged histogram.  Sets S.found[0],
    // S.fd[0], S.hc of that bin and, with rkt, the best race key above it
    // (S.sc64[0]).  Returns false (nothing set) when rounding leaves no such
    // bin in that chunk; the caller then merges every bin.
    auto chunk_bucket = [&](double need, bool rkt) -> bool {
        const uint32_t slot0 = qi * ntiles;
        // the bucket buffer is free here: the tiles' values gathered into it
        // with one load per thread, then summed per lane in tile order
        double *gs = reinterpret_cast<double *>(S.coll);  // [tile][FB_CHUNKS] or [tile][bin]
        uint64_t *gk = S.coll + FB_TILES_MAX * FB_CHUNKS;
        uint32_t *gc = reinterpret_cast<uint32_t *>(S.coll + 2 * FB_TILES_MAX * FB_CHUNKS);
        static_assert(FB_TILES_MAX * FB_CHUNKS * 5 / 2 <= K3_COLLECT, "gather scratch");
        for (int p = tid; p < (int)ntiles * FB_CHUNKS; p += K3_THREADS) {
            const FbPart pt = fb_part(W.fbpart, slot0 + (uint32_t)(p / FB_CHUNKS));
            gs[p] = pt.csum[p % FB_CHUNKS];
            gk[p] = pt.crk[p % FB_CHUNKS];
        }
        __syncthreads();
        const int lane = tid & 63;
        uint64_t ck = 0ull;  // wave 0: the chunk's largest race key
        if (tid < 64) {
            double cs = 0.0;
            for (uint32_t t = 0; t < ntiles; ++t) {
                cs += gs[t * FB_CHUNKS + lane];
                const uint64_t k = gk[t * FB_CHUNKS + lane];
                ck = k > ck ? k : ck;
            }
            // shuffles with every lane active (an inactive lane reads as 0)
            const double incl = wave_incl_scan_f64(cs, lane);
            const double excl = __shfl_up(incl, 1, 64);
            const uint64_t reach = __ballot(incl >= need);
            const int l = reach ? __builtin_ctzll(reach) : 0;
            const double excl_l = __shfl(excl, l, 64);
            if (lane == 0) {
                S.found[1] = reach ? (uint32_t)l : NONE;
                S.fd[1] = l == 0 ? 0.0 : excl_l;
            }
        }
        __syncthreads();
        const uint32_t lsel = S.found[1];
        if (lsel == NONE) return false;  // uniform
        const double acc0 = S.fd[1];
        __syncthreads();  // gs / gk reused below
        for (int p = tid; p < (int)ntiles * FB_CHUNK_BINS; p += K3_THREADS) {
            const FbPart pt = fb_part(W.fbpart, slot0 + (uint32_t)(p / FB_CHUNK_BINS));
            const int bin = K3_BINS - 1 - (int)lsel * FB_CHUNK_BINS - p % FB_CHUNK_BINS;
            gs[p] = pt.hm[bin];
            gc[p] = pt.hc[bin];
            gk[p] = pt.rk[bin];  // read whether or not written: used only with rkt
        }
        __syncthreads();
        if (tid < 64) {
            const int bin = K3_BINS - 1 - (int)lsel * FB_CHUNK_BINS - lane;
            double mb = 0.0;
            uint32_t cb = 0u;
            uint64_t kb = 0ull;
            if (lane < FB_CHUNK_BINS)
                for (uint32_t t = 0; t < ntiles; ++t) {
                    mb += gs[t * FB_CHUNK_BINS + lane];
                    cb += gc[t * FB_CHUNK_BINS + lane];
                    const uint64_t k = gk[t * FB_CHUNK_BINS + lane];
                    kb = k > kb ? k : kb;
                }
            const double bi = wave_incl_scan_f64(mb, lane);
            const double bi_up = __shfl_up(bi, 1, 64);
            const double acc = acc0 + (lane == 0 ? 0.0 : bi_up);
            const uint64_t hit = __ballot(lane < FB_CHUNK_BINS && mb > 0.0 && acc + mb >= need);
            const int tb = hit ? __builtin_ctzll(hit) : 0;
            // race keys of the chunks above and of the bins above it
            uint64_t top = (lane < (int)lsel ? ck : 0ull);
            const uint64_t kbin = lane < tb ? kb : 0ull;
            top = kbin > top ? kbin : top;
#pragma unroll
            for (int sft = 32; sft >= 1; sft >>= 1) {
                const uint64_t o = shx64(top, sft);
                top = o > top ? o : top;
            }
            if (hit && lane == tb) {
                S.found[0] = (uint32_t)bin;
                S.fd[0] = acc;
                S.hc[bin] = cb;
            }
            if (lane == 0) {
                if (rkt) S.sc64[0] = top;
                S.found[3] = hit ? 1u : 0u;
            }
        }
        __syncthreads();
        return S.found[3] != 0u;
    };

    // With pre (the first search of a tiled row) the first level's histogram
    // is the tiles' merged one, and its total mass pre_z.
    auto search = [&](double tval, bool frac, bool count, bool rk_on, bool pre, uint64_t &Tst,
                      double &ZKo) {
        double above = 0.0, target = 0.0;
        int nlev = 0;
        int path = 0;  // 1 collect, 2 ties
        uint32_t bsel = 0, bcnt = 0, bklo = 0, bkhi_sel = 0xffffffffu;
        for (int level = 0; level < 6; ++level) {
            // bin function of this level
            float lo = 0.0f, scale = 0.0f;
            uint32_t klo = 0, sh = 0;
            if (level == 0) {
                level0_bins(info.m, rowlo, cfloor, lo, scale);
            } else {
                klo = S.lv_klo[level];
                sh = S.lv_sh[level];
            }
            const bool rkl = rk_on && level == 0;
            const bool merged = pre && level == 0;
            if (!merged) {
                for (int i = tid; i < K3_BINS; i += K3_THREADS) {
                    S.hm[i] = 0.0;
                    S.hc[i] = 0u;
                    S.hlo[i] = NONE;
                    S.hhi[i] = 0u;
                    if (rkl) S.rk[i] = 0ull;
                }
                __syncthreads();
            }
            double zt = 0.0;
            auto visit = [&](float x, uint32_t j, float qj) {
                if ((!count && !(x > -INFINITY)) || mkcomp(x, j) < cfloor) return;
                uint32_t k = f2key(x);
                if (!in_play(S, x, k, nlev)) return;
                double e = count ? 1.0 : exp_neg_tab((double)x - m, S.etab);
                if (level == 0) zt += e;
                uint32_t bi = (level == 0) ? bin_value(x, lo, scale) : bin_key(k, klo, sh);
                atomicAdd(&S.hm[bi], e);
                atomicAdd(&S.hc[bi], 1u);
                if (level != 0) {  // level 0: the key range follows from the bin edges
                    atomicMin(&S.hlo[bi], k);
                    atomicMax(&S.hhi[bi], k);
                }
                if (rkl) atomicMax(&S.rk[bi], race_key(x, e, (double)qj + (double)P.eps, j));
            };
            if (merged) {
            } else if (rkl) {
                row_pass_q<DT, AL, XF>(P, b, S.bm, rowq, [&](float x, float qj, uint32_t j) {
                    visit(x, j, qj);
                });
            } else {
                row_pass<DT, AL, XF>(P, b, S.bm, [&](float x, uint32_t j) { visit(x, j, 0.0f); });
            }
            if (level == 0) {
                const double Z = merged ? pre_z : wg_sum_f64<K3_THREADS>(zt, S.scd);
                target = frac ? tval * Z : tval;
            }
            bool quick = false;  // the bucket found from the tiles' chunk summaries
            if (merged) {
                quick = chunk_bucket(target - above, rkl);
                if (quick && rkl) rk_top = S.sc64[0];
                if (!quick) merge_parts(rkl);
            }
            if (!quick) find_bucket(S.hm, S.hc, target - above, S.lane_sum, S.found, S.fd);
            const uint32_t fb = S.found[0];
            const double bbefore = S.fd[0];
            if (rkl && !quick) {
                // the best key of the bins above the boundary (all of them in K)
                uint64_t t = 0;
                for (int i = tid; i < K3_BINS; i += K3_THREADS)
                    if ((uint32_t)i > fb && S.rk[i] > t) t = S.rk[i];
                rk_top = wg_max_u64<K3_THREADS>(t, S.sc64);
            }
            __syncthreads();
            above += bbefore;
            bsel = fb;
            bcnt = S.hc[fb];
            if (merged && tid == 0) {
                // the waiting tiles collect this bucket (or nothing)
                __hip_atomic_store(&W.fbsync[(size_t)qi * FB_SYNC_WORDS + 1],
                                   bcnt <= (uint32_t)K3_COLLECT ? fb + 1u : FB_NO_BUCKET,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            bklo = S.hlo[fb];
            uint32_t bkhi = S.hhi[fb];
            if (level == 0) level0_keys(fb, lo, scale, info.m, bklo, bkhi);
            bkhi_sel = bkhi;
            __syncthreads();
            if (tid == 0) {
                if (level == 0) {
                    S.lv_lo = lo;
                    S.lv_scale = scale;
                }
                S.lv_bin[level] = fb;
                if (level + 1 < 8) {
                    S.lv_klo[level + 1] = bklo;
                    S.lv_sh[level + 1] = bin_shift((uint64_t)(bkhi - bklo) + 1ull);
                }
            }
            __syncthreads();
            nlev = level + 1;
            if (bcnt <= (uint32_t)K3_COLLECT) {
                path = 1;
                break;
            }
            if (bklo == bkhi) {
                path = 2;
                break;
            }
        }
        (void)bsel;
        if (path == 0) path = 1;  // unreachable: a key range of 1 is reached by level 4
        const bool rk_level0 = rk_on && nlev == 1 && path == 1;
        if (path == 1) {
            if (tid == 0) S.counter = 0;
            __syncthreads();
            // the bucket's members lie in its key range [bklo, bkhi_sel]
            auto collect = [&](float x, uint32_t j) {
                if ((!count && !(x > -INFINITY)) || mkcomp(x, j) < cfloor) return;
                uint32_t k = f2key(x);
                if (!in_play(S, x, k, nlev)) return;
                uint32_t pos = atomicAdd(&S.counter, 1u);
                if (pos < (uint32_t)K3_COLLECT) S.coll[pos] = mkcomp(x, j);
            };
            bool whole_row = true;
            if (pre && nlev == 1) {
                // the bucket was published: this tile collects its own range
                // while the others collect theirs, then their lists follow
                // its own in coll (at most FB_POLLS polls for them)
                const int c0 = (int)tile * ft.TL, c1 = min(c0 + ft.TL, P.V);
                key_scan<DT, AL, XF>(P, b, c0, c1, bklo, bkhi_sel, S.bm, collect);
                uint32_t *sy = W.fbsync + (size_t)qi * FB_SYNC_WORDS;
                if (tid == 0) {
                    uint32_t d = 0u;
                    for (int it = 0; it < FB_POLLS; ++it) {
                        d = __hip_atomic_load(&sy[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (d >= ntiles - 1) break;
                        __builtin_amdgcn_s_sleep(8);
                    }
                    uint32_t nl = NONE;
                    if (d >= ntiles - 1) {
                        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                        nl = __hip_atomic_load(&sy[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    S.found[1] = nl;
                }
                __syncthreads();
                const uint32_t nl = S.found[1];
                if (nl != NONE) {
                    const uint32_t own = min(S.counter, (uint32_t)K3_COLLECT);
                    const uint64_t *mem = fb_members(W.fbpart, qi * ntiles);
                    for (uint32_t i = tid; i < nl; i += K3_THREADS)
                        if (own + i < (uint32_t)K3_COLLECT) S.coll[own + i] = mem[i];
                    __syncthreads();
                    if (tid == 0) S.counter = own + nl;
                    __syncthreads();
                    whole_row = false;
                } else {
                    if (tid == 0) S.counter = 0;  // gave up: the whole row below
                    __syncthreads();
                }
            }
            if (whole_row) key_scan<DT, AL, XF>(P, b, 0, P.V, bklo, bkhi_sel, S.bm, collect);
            const int n = (int)min(S.counter, (uint32_t)K3_COLLECT);
            uint32_t fi;
            if (n <= K3_THREADS) {
                // one member per thread: sorted in registers, masses and
                // their running sum from the top (above + the members before
                // it + its own) one per thread
                const int npad = pow2_ceil(n < 1 ? 1 : n);
                uint64_t c = tid < n ? S.coll[tid] : 0ull;
                __syncthreads();
                c = bitonic_regs_desc(c, npad, S.coll);
                if (tid < n) S.coll[tid] = c;
                const double e1 = tid < n ? (count ? 1.0 : exp_neg_tab((double)cval(c) - m, S.etab)) : 0.0;
                double tot;
                const double run = (above + wg_excl_scan_f64<K3_THREADS>(e1, S.scd, tot)) + e1;
                fi = wg_min_u32<K3_THREADS>(tid < n && run >= target ? (uint32_t)tid : NONE, S.sc);
                if (fi == NONE) fi = (uint32_t)(n > 0 ? n - 1 : 0);  // rounding: whole bucket
                // ZK: mass of every kept element = the running sum through fi
                if (tid == (int)fi) S.fd[1] = n > 0 ? run : above;
                __syncthreads();
                ZKo = S.fd[1];
            } else {
                const int npad = pow2_ceil(n);
                for (int i = n + tid; i < npad; i += K3_THREADS) S.coll[i] = 0ull;
                __syncthreads();
                bitonic_desc<K3_THREADS>(S.coll, npad);
                // masses of the sorted bucket members, 4 per thread
                constexpr int PER = K3_COLLECT / K3_THREADS;
                double ei[PER];
                double loc = 0.0;
#pragma unroll
                for (int t = 0; t < PER; ++t) {
                    int i = tid * PER + t;
                    ei[t] = (i < n) ? (count ? 1.0 : exp_neg_tab((double)cval(S.coll[i]) - m, S.etab)) : 0.0;
                    loc += ei[t];
                }
                double tot;
                double run = above + wg_excl_scan_f64<K3_THREADS>(loc, S.scd, tot);
                uint32_t first = NONE;
#pragma unroll
                for (int t = 0; t < PER; ++t) {
                    int i = tid * PER + t;
                    run += ei[t];
                    if (i < n && first == NONE && run >= target) first = (uint32_t)i;
                }
                fi = wg_min_u32<K3_THREADS>(first, S.sc);
                if (fi == NONE) fi = (uint32_t)(n - 1);  // rounding: whole bucket
                // ZK: mass of every kept element = above + bucket prefix through fi
                double sk = 0.0;
#pragma unroll
                for (int t = 0; t < PER; ++t) {
                    int i = tid * PER + t;
                    if (i <= (int)fi && i < n) sk += ei[t];
                }
                ZKo = above + wg_sum_f64<K3_THREADS>(sk, S.scd);
            }
            Tst = (n > 0) ? S.coll[fi] : mkcomp(info.m, info.idx0);
            if (rk_level0 && n > 0) {
                rk_done = true;
                rk_fi = fi;
            }
        } else {
            // every bucket member has the same value: take the c members with
            // the smallest vocab ids
            const float xt = key2f(bklo);
            const double et = count ? 1.0 : exp_neg_tab((double)xt - m, S.etab);
            double cnt_need = ceil((target - above) / et);
            uint32_t cneed = (cnt_need < 1.0) ? 1u : (cnt_need > (double)bcnt ? bcnt : (uint32_t)cnt_need);
            // c-th smallest index among elements equal to xt: scan in index order
            const void *rowp = row_ptr(P, DT, b);
            uint32_t seen = 0;  // uniform running count
            if (tid == 0) S.found[1] = NONE;
            __syncthreads();
            for (int64_t s0 = 0; s0 < P.V && S.found[1] == NONE; s0 += K3_SEG) {
                const int64_t s1 = min(s0 + (int64_t)K3_SEG, (int64_t)P.V);
                if (P.pen) build_bitmap<K3_THREADS>(S.bm, s0, s1 - s0, P, b);
                for (int64_t t0 = s0; t0 < s1; t0 += (int64_t)K3_THREADS * VEC) {
                    int64_t j = t0 + (int64_t)tid * VEC;
                    int64_t rem = s1 - j;
                    int nv = rem <= 0 ? 0 : (rem >= 8 ? 8 : (int)rem);
                    float x[8];
                    load8<DT, AL>(rowp, j, nv, x);
                    uint32_t bits = 0;
                    if (P.pen && nv > 0) {
                        int64_t r = j - s0;
                        bits = (S.bm[r >> 5] >> (r & 31)) & 0xffu;
                    }
                    uint32_t mm = 0;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        if (i < nv && xform<XF>(x[i], (bits >> i) & 1u, P) == xt) mm |= 1u << i;
                    uint32_t tot;
                    uint32_t off = wg_excl_scan_u32<K3_THREADS>(__popc(mm), S.sc, tot);
                    if (seen + off < cneed && cneed <= seen + off + __popc(mm)) {
                        uint32_t r = cneed - (seen + off);  // r-th set bit (1-based)
                        for (int i = 0; i < 8; ++i)
                            if ((mm >> i) & 1u) {
                                if (--r == 0) {
                                    S.found[1] = (uint32_t)(j + i);
                                    break;
                                }
                            }
                    }
                    seen += tot;
                    __syncthreads();
                    if (S.found[1] != NONE) break;
                }
                __syncthreads();
            }
            Tst = mkcomp(xt, S.found[1]);
            ZKo = above + (double)cneed * et;
        }
    };

    // Up to three searches, from one call site: (0) for a top-k row without a
    // known floor, its kk-th element by count, which becomes the floor (its
    // value, when ties are kept); (1) the top-p cut at p -- or, for a row
    // queued only for an inverse-CDF draw over the whole row, that draw at u;
    // (2) the draw inside the cut at u ZK.  A level <= 0 (or NaN) stands for
    // the first element of the order.
    const uint64_t top = mkcomp(info.m, info.idx0);
    uint64_t Tstar = top;  // the cut (or the whole-row draw)
    double ZK = 1.0;       // mass of the cut, exp(x - m) summed
    uint64_t Tdraw = top;  // the draw inside the cut
    for (int job = 0; job < 3; ++job) {
        double tval;
        bool frac, count = false;
        if (job == 0) {
            if (whole || !md.tk || cfloor != 0) continue;
            tval = (double)md.k;
            frac = false;
            count = true;
        } else if (job == 1) {
            if (!whole && !md.tp) {
                // top-k alone: the cut is the floor
                Tstar = cfloor;
                double z = 0.0;
                row_pass<DT, AL, XF>(P, b, S.bm, [&](float x, uint32_t j) {
                    if (mkcomp(x, j) >= cfloor) z += exp_neg_tab((double)x - m, S.etab);
                });
                ZK = wg_sum_f64<K3_THREADS>(z, S.scd);
                continue;
            }
            const double level = whole ? (double)P.u[b] : (double)md.p;
            if (!(level > 0.0)) continue;
            tval = level;
            frac = true;
        } else {
            if (whole || !md.inv || !(P.u[b] > 0.0f)) break;
            tval = (double)P.u[b] * ZK;
            frac = false;
        }
        uint64_t Tj;
        double Zj;
        search(tval, frac, count, job == 1 && md.sm && !whole, job == 1 && pre0, Tj, Zj);
        if (job == 0) {
            cfloor = (P.flags & TOPK_TIES) ? (Tj >> 32) << 32 : Tj;
        } else if (job == 1) {
            Tstar = Tj;
            ZK = Zj;
        } else {
            Tdraw = Tj < Tstar ? Tstar : Tj;  // inside the cut whatever the rounding
        }
    }
    if (whole) {
        if (tid == 0) P.out_idx[b] = (int64_t)cidx(Tstar);
        __syncthreads();  // the next row reuses the shared buffers
        continue;
    }

    // ---- exponential race over K = { comp >= T* }, or greedy
    uint32_t idx = info.idx0;
    if (md.sm && rk_done) {
        // K = the bins above the boundary (their best key) and the bucket's
        // sorted members 0 .. rk_fi: the winner over both, ratios in double
        double rr = -1.0;
        uint32_t ri = NONE;
        for (uint32_t i = tid; i <= rk_fi; i += K3_THREADS) {
            const uint64_t c = S.coll[i];
            const uint32_t id = cidx(c);
            const float x = cval(c);
            const double r = race_ratio(x, exp_neg_tab((double)x - m, S.etab), (double)rowq[id] + (double)P.eps);
            if (r > rr || (r == rr && id < ri)) {
                rr = r;
                ri = id;
            }
        }
        if (rk_top != 0ull) {
            // the key's candidate (the same id in every thread): its logit
            // read again and transformed, the history searched by the whole
            // workgroup for its penalty
            const uint32_t id = race_key_id(rk_top);
            int hit = 0;
            if (XF && P.pen) {
                const int64_t i0 = P.offsets[b];
                int64_t i1 = P.offsets[b + 1];
                if (P.plen) {
                    const int64_t n = P.plen[b] < 0 ? 0 : P.plen[b];
                    if (i0 + n < i1) i1 = i0 + n;
                }
                for (int64_t h = i0 + tid; h < i1; h += K3_THREADS) hit |= P.ids[h] == (int32_t)id;
            }
            hit = __syncthreads_or(hit);
            if (tid == 0) {
                const float x = xform<XF>(ld1<DT>(row_ptr(P, DT, b), id), hit ? 1u : 0u, P);
                const double r =
                    race_ratio(x, exp_neg_tab((double)x - m, S.etab), (double)rowq[id] + (double)P.eps);
                if (r > rr || (r == rr && id < ri)) {
                    rr = r;
                    ri = id;
                }
            }
        }
        idx = wg_best_ratio<K3_THREADS>(rr, ri, S.scd, S.sci);
    } else if (md.sm) {
        Race rc;
        rc.x = -INFINITY; rc.qe = 1.0f; rc.idx = NONE; rc.lq = 0.0f;
        const float *rowq = P.q + (int64_t)b * P.V;
        row_pass_q<DT, AL, XF>(P, b, S.bm, rowq, [&](float x, float qj, uint32_t j) {
            if (mkcomp(x, j) >= Tstar) race_offer(rc, x, qj + P.eps, j);
        });
        Race r = wg_race<K3_THREADS>(rc, S.scx, S.scq, S.sci);
        idx = r.idx;
    } else if (md.inv) {
        idx = cidx(Tdraw);
    }
    if (tid == 0) {
        P.out_idx[b] = (int64_t)idx;
        info.kind = KIND_THRESH;
        info.T = Tstar;
        info.ZK = ZK;
        W.info[b] = info;
    }
    __syncthreads();  // the next row reuses the shared buffers
    }
}

// ================================================================== k_dense

// Dense outputs of one dense tile of one row, in whole lines: the filtered
// logits of rows with top-k / top-p (x at the kept ids, -inf elsewhere; rows
// without a filter got theirs from the pass) and, when asked for, the
// probabilities (pi at the kept ids, 0 elsewhere).  A dense tile is
// DGR_PER_TILE group-rows of DGR elements spaced ntd group-rows apart: group-
// row g of the row belongs to tile g mod ntd.  Spreading a workgroup's
// stores over the row in this way writes faster than one contiguous span per
// workgroup.  Rows with a kept list compose the tile in LDS (-inf, then each
// kept value at its place) without reading the logits; threshold rows (after
// the full-row search) and unfiltered rows re-read the tile's logits.

// tv first and 16-byte aligned, so that its vector accesses compile to
// single 16-byte LDS operations (two 8-byte halves conflict on the banks).
struct alignas(16) DenseShared {
    float tv[DTILE];            // a listed row's tile, composed
    double etab[64];            // exp2_j64_tab (probabilities only)
    uint32_t tb[DTILE / 32];    // penalised positions of the tile (threshold rows)
};

static_assert(DGR == 8 * DENSE_THREADS, "a group-row is two vectors of 4 floats per lane");

// What a dense tile needs before its stores: the row's kind and the range of
// the kept list, requested one tile ahead.
struct DenseMeta {
    RowInfo info;
    uint32_t k0, k1;
};

__device__ __forceinline__ DenseMeta dense_meta(const KParams &P, const KWork &W, int ntd, int i) {
    const int b = P.b0 + i / ntd, t = i % ntd;
    const uint32_t *kto = W.ktoff + (int64_t)b * (ntd + 1);
    DenseMeta dm;
    dm.info = W.info[b];
    dm.k0 = kto[t];
    dm.k1 = kto[t + 1];
    return dm;
}

// One dense tile: tile t of row b, metadata dm.
template <int DT, bool AL, bool XF>
__device__ __forceinline__ void dense_tile_write(const KParams &P, const KWork &W, int ntd, int b,
                                                 int t, const DenseMeta &dm, DenseShared &S) {
    constexpr int NT = DENSE_THREADS;
    const int tid = threadIdx.x;
    const int ngr = (P.V + DGR - 1) / DGR;
    const RowInfo &info = dm.info;
    float *ol = (P.out_logits && info.kind != KIND_UNFILTERED)
                    ? P.out_logits + (int64_t)b * P.V : nullptr;
    float *op = P.out_probs ? P.out_probs + (int64_t)b * P.V : nullptr;
    if (!ol && !op) return;
    const double m = (double)info.m, ZK = info.ZK;
    constexpr int NW = DTILE / 32;  // bitmap words

    if (info.kind == KIND_LIST) {
        const int k0 = (int)min(dm.k0, (uint32_t)KMAX);
        const int k1 = (int)min(max(dm.k1, (uint32_t)k0), (uint32_t)KMAX);
        const uint64_t *kl = W.klist + (int64_t)b * KMAX;
        // the tile's kept entries (the merge grouped them by dense tile), at
        // most KMAX / NT per thread
        constexpr int KR = KMAX / NT;
        uint64_t kv[KR];
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            const int i = k0 + r * NT + tid;
            kv[r] = i < k1 ? kl[i] : 0ull;
        }
        // the tile composed in LDS: -inf everywhere, then each kept value at
        // its place
        static_assert(DTILE % (4 * NT) == 0, "the fill is whole vectors per thread");
        const f32x4 ninf = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int w = tid; w < DTILE / 4; w += NT) reinterpret_cast<f32x4 *>(S.tv)[w] = ninf;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < KR; ++r)
            if (k0 + r * NT + tid < k1) S.tv[dense_pos(cidx(kv[r]), (uint32_t)ntd)] = cval(kv[r]);
        __syncthreads();
        // each lane writes the 4 floats at 4 tid and the 4 at DGR/2 + 4 tid of
        // each group-row, so that a wave's store covers 1 KB without gaps (as
        // the pass's stores do)
#pragma unroll
        for (int i = 0; i < DGR_PER_TILE; ++i) {
            const int g = t + i * ntd;
            if (g >= ngr) break;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = i * DGR + h * (DGR / 2) + 4 * tid;
                const int j = g * DGR + h * (DGR / 2) + 4 * tid;
                const int nv = nv4(j, P.V);
                if (nv == 0) continue;
                const f32x4 a = *reinterpret_cast<const f32x4 *>(S.tv + r);
                const float xv[4] = {a[0], a[1], a[2], a[3]};
                if (ol) store4<AL>(ol, j, nv, xv);
                if (op) {
                    float o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[e] = xv[e] > -INFINITY ? (float)(exp_neg_tab((double)xv[e] - m, S.etab) / ZK)
                                                 : 0.0f;
                    store4<AL>(op, j, nv, o);
                }
            }
        }
        return;
    }
    if (info.kind != KIND_THRESH && info.kind != KIND_UNFILTERED) return;
    // K = { comp >= T } (T = 0 keeps the whole row): re-read the tile
    if (XF && P.pen) {
        // the tile's penalised positions
        for (int w = tid; w < NW; w += NT) S.tb[w] = 0u;
        __syncthreads();
        const int64_t i0 = P.offsets[b];
        int64_t i1 = P.offsets[b + 1];
        if (P.plen) {
            const int64_t n = P.plen[b] < 0 ? 0 : P.plen[b];
            if (i0 + n < i1) i1 = i0 + n;
        }
        for (int64_t h = i0 + tid; h < i1; h += NT) {
            const int32_t id = P.ids[h];
            if (id >= 0 && id < P.V && dense_tile((uint32_t)id, (uint32_t)ntd) == (uint32_t)t) {
                const uint32_t rr = dense_pos((uint32_t)id, (uint32_t)ntd);
                atomicOr(&S.tb[rr >> 5], 1u << (rr & 31));
            }
        }
        __syncthreads();
    }
    const void *rowp = row_ptr(P, DT, b);
    const uint64_t T = info.T;
#pragma unroll
    for (int i = 0; i < DGR_PER_TILE; ++i) {
        const int g = t + i * ntd;
        if (g >= ngr) break;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = i * DGR + h * (DGR / 2) + 4 * tid;
            const int j = g * DGR + h * (DGR / 2) + 4 * tid;
            const int nv = nv4(j, P.V);
            if (nv == 0) continue;
            Raw4<DT> raw;
            load4<DT, AL>(rowp, j, nv, raw);
            float x[4];
            unpack4<DT>(raw, x);
            const uint32_t bits = (XF && P.pen) ? (S.tb[r >> 5] >> (r & 31)) & 0xfu : 0u;
            float lo[4], po[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float xi = xform<XF>(x[e], (bits >> e) & 1u, P);
                const bool in = mkcomp(xi, (uint32_t)(j + e)) >= T;
                lo[e] = in ? xi : -INFINITY;
                po[e] = in ? (float)(exp_neg_tab((double)xi - m, S.etab) / ZK) : 0.0f;
            }
            if (ol) store4<AL>(ol, j, nv, lo);
            if (op) store4<AL>(op, j, nv, po);
        }
    }
    if (XF && P.pen) __syncthreads();  // the next tile rewrites the bitmap
}

// One dense tile per workgroup, B x ntd of them.
template <int DT, bool AL, bool XF>
__global__ __launch_bounds__(DENSE_THREADS) void k_dense(KParams P, KPlan L, KWork W) {
    __shared__ DenseShared S;
    const int ntd = L.ntd;
    const int i = (int)blockIdx.x;
    if (P.out_probs) {  // the same for the whole grid
        if (threadIdx.x < 64) S.etab[threadIdx.x] = exp2_j64_tab[threadIdx.x];
        __syncthreads();
    }
    dense_tile_write<DT, AL, XF>(P, W, ntd, P.b0 + i / ntd, i % ntd, dense_meta(P, W, ntd, i), S);
}

// ================================================================== k_epilogue
// The decode-step epilogue, in the order of the MiniMind loop (sec. 10.9):
// force EOS on finished rows, mark rows whose output is EOS, append the
// output to the history (the loop's concatenation onto the sequence), count
// the rows still running (the loop's all-finished test).  One workgroup
// strides over every row of the call, so the counts need no zeroed memory
// and no atomics.
__global__ __launch_bounds__(EPI_THREADS) void k_epilogue(EpiParams E) {
    __shared__ uint32_t red[2][EPI_THREADS / 64];
    uint32_t unf = 0, full = 0;
    for (int b = threadIdx.x; b < E.B; b += EPI_THREADS) {
        int64_t t = E.out_idx[b];
        if (E.finished) {
            uint8_t f = E.finished[b];
            if (f) {
                t = E.eos;
                E.out_idx[b] = t;
            } else if (t == E.eos) {
                f = 1;
                E.finished[b] = f;
            }
            unf += f == 0;
        } else {
            ++unf;
        }
        if (E.append) {
            const int64_t i0 = E.offsets[b], cap = E.offsets[b + 1] - i0;
            const int64_t n = E.len[b] < 0 ? 0 : E.len[b];
            if (n < cap) {
                E.ids[i0 + n] = (int32_t)t;
                E.len[b] = (int32_t)(n + 1);
            } else {
                ++full;
            }
        }
    }
    unf = wave_sum_u32(unf);
    full = wave_sum_u32(full);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[0][w] = unf;
        red[1][w] = full;
    }
    __syncthreads();
    if (threadIdx.x == 0 && E.counts) {
        uint32_t a = 0, c = 0;
        for (int i = 0; i < EPI_THREADS / 64; ++i) {
            a += red[0][i];
            c += red[1][i];
        }
        E.counts[0] = (int32_t)a;
        E.counts[1] = (int32_t)c;
    }
}

template <class K>
hipError_t launch(K kern, dim3 grid, dim3 block, size_t shmem, hipStream_t s, const KParams &p,
                  const KPlan &l, const KWork &w) {
    if (grid.x == 0) return hipSuccess;
    hipLaunchKernelGGL(kern, grid, block, shmem, s, p, l, w);
    return hipGetLastError();
}

}  // namespace

// Instantiation table: storage type x 16-byte-aligned rows x transform stage
// (penalty or temperature present).
#define SMP_PICK(KERN, grid, block, shmem)                                                 \
    (xf ? (dtype == 1 ? (al ? launch(KERN<1, true, true>, grid, block, shmem, s, p, l, w)   \
                            : launch(KERN<1, false, true>, grid, block, shmem, s, p, l, w)) \
                      : (al ? launch(KERN<0, true, true>, grid, block, shmem, s, p, l, w)   \
                            : launch(KERN<0, false, true>, grid, block, shmem, s, p, l, w)))\
        : (dtype == 1 ? (al ? launch(KERN<1, true, false>, grid, block, shmem, s, p, l, w)  \
                            : launch(KERN<1, false, false>, grid, block, shmem, s, p, l, w))\
                      : (al ? launch(KERN<0, true, false>, grid, block, shmem, s, p, l, w)  \
                            : launch(KERN<0, false, false>, grid, block, shmem, s, p, l, w))))

static bool any_transform(const KParams &p) { return p.pen || p.temperature != 1.0f; }

hipError_t launch_plan(const KParams &p, const KPlan &l, const KWork &w, int dtype, bool al,
                       hipStream_t s) {
    const bool xf = any_transform(p);
    dim3 grid((unsigned)p.B), block(K1_THREADS);
    return SMP_PICK(k_plan, grid, block, 0);
}

hipError_t launch_pass(const KParams &p, const KPlan &l, const KWork &w, int dtype, bool al,
                       hipStream_t s) {
    const bool xf = any_transform(p);
    dim3 grid((unsigned)((int64_t)p.B * l.nt)), block(PASS_THREADS);
    size_t sh = p.pen ? (size_t)((l.seg + 31) / 32) * 4 : 0;
    static_assert(sizeof(Raw4<0>) * PASS_WAVES * PASS_D_MAX * 64 + (SEG_MAX / 32) * 4 <= 65536,
                  "pass LDS: staging and the penalty bitmap of the longest tile");
    return SMP_PICK(k_pass, grid, block, sh);
}

hipError_t launch_rows(const KParams &p, const KPlan &l, const KWork &w, hipStream_t s) {
    // per-sub-slot candidate offsets, then per-dense-tile counts of the kept list
    static_assert(PASS_WAVES == 4, "rows_lds_words counts four sub-slots per tile");
    // the largest dynamic part is that of the longest row at the shortest tile
    static_assert(sizeof(RowsShared) + 4 * rows_lds_words(make_plan(SAMPLER_VOCAB_MAX, SEG_MIN, 1)) <=
                      65536,
                  "row merge LDS");
    const size_t sh = (size_t)rows_lds_words(l) * 4;
    return launch(k_rows, dim3((unsigned)p.B), dim3(ROWS_THREADS), sh, s, p, l, w);
}

hipError_t launch_fallback(const KParams &p, const KPlan &l, const KWork &w, int dtype, bool al,
                           hipStream_t s) {
    const bool xf = any_transform(p);
    // one workgroup per CU (its LDS allows no more); queued rows (or their
    // tiles) are spread over them, none queued costs one read per workgroup
    dim3 grid((unsigned)fb_grid(p.B)), block(K3_THREADS);
    return SMP_PICK(k_fallback, grid, block, 0);
}

hipError_t launch_dense(const KParams &p, const KPlan &l, const KWork &w, int dtype, bool al,
                        hipStream_t s) {
    const bool xf = any_transform(p);
    dim3 grid((unsigned)((int64_t)p.B * l.ntd)), block(DENSE_THREADS);
    return SMP_PICK(k_dense, grid, block, 0);
}

#undef SMP_PICK

// The workspace of sampler_run_static: one array per device, in the code
// object's device memory, held until the process ends.  Host code must not
// pass `scratch` itself to a kernel (in host code the name is a stand-in, not
// a device address); static_scratch looks the device address up once per
// device and every use goes through that address.
static __device__ __align__(256) unsigned char scratch[SAMPLER_STATIC_SCRATCH_BYTES];

namespace {
constexpr int SCRATCH_DEVICES = 64;
void *scratch_addr[SCRATCH_DEVICES];
std::mutex scratch_mu;
}  // namespace

hipError_t static_scratch(int device, void **ptr) {
    if (device < 0 || device >= SCRATCH_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_addr[device] == nullptr) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        scratch_addr[device] = p;
    }
    *ptr = scratch_addr[device];
    return hipSuccess;
}

hipError_t launch_epilogue(const EpiParams &e, hipStream_t s) {
    hipLaunchKernelGGL(k_epilogue, dim3(1), dim3(EPI_THREADS), 0, s, e);
    return hipGetLastError();
}

}  // namespace smp
