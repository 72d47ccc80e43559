// HIP kernels of the batched logits sampler (gfx950, wave64).
//
// Pipeline of one call (all on the caller's stream):
//
//   k_chunk     grid = B x nch.  One workgroup streams one chunk of one row
//               once from HBM: widen bf16 -> fp32, repetition penalty (LDS
//               bitmap of the chunk's history ids), temperature.  Depending on
//               the row's stages it then
//                 - keeps the chunk's top-kk candidates in an LDS buffer
//                   filtered by a rising threshold (the rolling top-k of the
//                   Ascend npu_top_k_top_p_sample page, topK section: each
//                   batch of elements is prefiltered by the k-th value of
//                   what came before, the buffer is cut back to exactly kk by
//                   a radix select when it fills);
//                 - accumulates the chunk's max / sum-exp for top-p rows
//                   without top-k (the softmax of that page's topP section);
//                 - runs the exponential race over the whole chunk for rows
//                   that only sample (streams q in the same pass);
//                 - writes the dense output of unfiltered rows.
//   k_rows      grid = B.  Merges the <= 8 chunk results of a row: exact
//               top-kk by radix select, bitonic sort, softmax in double,
//               inclusive scan, shortest prefix reaching p, exponential race
//               over the kept set (gather of q at the kept ids), output id.
//               Rows whose guess does not settle top-p are flagged.
//   k_fallback  grid = B (flagged rows only).  Full-row top-p cutoff: a
//               value-space mass histogram, then key-space refinement, then
//               an exact sort of the boundary bucket in LDS (or a rank among
//               ties by vocab id), then the race over the kept set.  This is
//               the page's full-sort fallback reached without a full sort.
//   k_dense     grid = B x tiles.  Writes the dense filtered logits (and the
//               optional probabilities) of filtered rows with full-line
//               stores, composing each tile in LDS from the kept list.
//
// Order and keys: a transformed logit x and its vocab id j form the 64-bit
// composite  (orderkey(x) << 32) | ~j ; larger composite = earlier in the
// row's order (larger value, then smaller id).  All composites of a row are
// distinct, so every selection below is exact and deterministic.

#include <math.h>
#include <stdint.h>

#include "sampler_internal.h"

namespace smp {
namespace {

constexpr uint32_t NONE = 0xffffffffu;
constexpr uint32_t NEED_LOGITS = 1u;
constexpr uint32_t NEED_PROBS = 2u;
// top-p decisions taken from a guess must clear the cutoff by this much
// (relative to the row's total mass); the row's total is accumulated from
// fp32 exponentials, good to about 1e-6.  Rows inside the margin take the
// exact full-row search.
constexpr double GUESS_MARGIN = 1e-5;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
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
    bool tk, tp, sm;
    int k;
    float p;
};

__device__ __forceinline__ Mode row_mode(const KParams &P, int b) {
    Mode md;
    uint32_t rf = P.row_flags ? (uint32_t)P.row_flags[b] : 7u;
    int kmax = P.V < KMAX ? P.V : KMAX;
    md.k = 0;
    md.p = 1.0f;
    md.tk = false;
    if ((rf & 1u) && P.top_k) {
        int k = P.top_k[b];
        if (k >= 1 && k <= kmax) {
            md.tk = true;
            md.k = k;
        }
    }
    md.tp = false;
    if ((rf & 2u) && P.top_p) {
        float p = P.top_p[b];
        if (p < 1.0f) {  // NaN compares false: stage off
            md.tp = true;
            md.p = p;
        }
    }
    md.sm = (rf & 4u) && P.q;
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

// Penalty bits of the 8 elements starting at row-relative offset r (a
// multiple of 8) of a bitmap that starts at offset 0.
template <bool XF>
__device__ __forceinline__ uint32_t pen_bits(const uint32_t *bm, int r, const KParams &P) {
    if (!XF || !P.pen) return 0u;
    return (bm[r >> 5] >> (r & 31)) & 0xffu;
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

// Plain write-back stores: each lane writes 32 contiguous bytes as two 16-byte
// stores, and L2 merges the two half lines of a wave before they reach HBM
// (streaming stores of half lines write at a fraction of the bandwidth).
template <bool AL>
__device__ __forceinline__ void store8(float *p, int64_t j, int nv, const float (&x)[8]) {
    if (AL && nv == 8) {
        f32x4 a = {x[0], x[1], x[2], x[3]};
        f32x4 c = {x[4], x[5], x[6], x[7]};
        *(f32x4 *)(p + j) = a;
        *((f32x4 *)(p + j) + 1) = c;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < nv) p[j + i] = x[i];
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
__device__ __forceinline__ float shxf(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ double shxd(double v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t t = (uint32_t)__shfl_up((int)v, d, 64);
        if (lane >= d) v += t;
    }
    return v;
}
__device__ __forceinline__ double wave_incl_scan_f64(double v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        double t = __shfl_up(v, d, 64);
        if (lane >= d) v += t;
    }
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
    for (int m = 32; m >= 1; m >>= 1) v += shxd(v, m);
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
        uint64_t o = shx64(v, m);
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
        uint64_t o = shx64(v, m);
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
    for (int m = 32; m >= 1; m >>= 1) v = min(v, shx(v, m));
    if ((threadIdx.x & 63) == 0) sc[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t t = NONE;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) t = min(t, sc[i]);
    __syncthreads();
    return t;
}

// Exponential race: is candidate a (logit xa, q+eps qa) ahead of b?
// e_a / qa > e_b / qb  <=>  exp(xa - xb) * qb > qa.  Equal -> smaller id.
struct Race {
    float x, qe;
    uint32_t idx;
};
// The exponentials use the hardware exp2 (relative error ~1e-6 where the
// two logits are far apart, where the comparison is never close).
__device__ __forceinline__ bool race_ahead(const Race &a, const Race &b) {
    if (a.idx == NONE) return false;
    if (b.idx == NONE) return true;
    float f = __expf(a.x - b.x) * b.qe;
    if (f > a.qe) return true;
    if (f < a.qe) return false;
    return a.idx < b.idx;
}
__device__ __forceinline__ void race_offer(Race &best, float x, float qe, uint32_t j) {
    if (!(x > -INFINITY)) return;  // probability 0: never drawn
    if (best.idx == NONE || __expf(x - best.x) * best.qe > qe) {
        best.x = x;
        best.qe = qe;
        best.idx = j;
    }
}
template <int NT>
__device__ __forceinline__ Race wg_race(Race r, float *scx, float *scq, uint32_t *sci) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        Race o;
        o.x = shxf(r.x, m);
        o.qe = shxf(r.qe, m);
        o.idx = shx(r.idx, m);
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
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) {
        Race o;
        o.x = scx[i];
        o.qe = scq[i];
        o.idx = sci[i];
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
        uint32_t S = s;  // suffix sum over lanes >= lane
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            uint32_t t = (uint32_t)__shfl_down((int)S, d, 64);
            if (lane + d < 64) S += t;
        }
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

// Radix select over distinct 64-bit composites held in registers.  Finds
// (prefix, pmask) such that exactly kk of the valid entries satisfy
// (v & pmask) >= prefix, i.e. the kk largest.  The bits all entries share
// are skipped first (min/max reduction), then digits of up to 8 bits are
// taken from the highest differing bit down, stopping as soon as the
// boundary bucket is taken whole.  Needs 1 <= kk < number of valid entries.
template <int NT, int R>
__device__ void wg_radix_select(const uint64_t (&v)[R], uint32_t vmask, uint32_t kk,
                                uint32_t *hist, uint32_t *sel, uint64_t *sc64,
                                uint64_t &prefix_out, uint64_t &pmask_out) {
    uint64_t mn = ~0ull, mx = 0ull;
#pragma unroll
    for (int r = 0; r < R; ++r)
        if ((vmask >> r) & 1u) {
            mn = v[r] < mn ? v[r] : mn;
            mx = v[r] > mx ? v[r] : mx;
        }
    mn = wg_min_u64<NT>(mn, sc64);
    mx = wg_max_u64<NT>(mx, sc64);
    const uint64_t diff = mn ^ mx;
    if (diff == 0) {
        prefix_out = mx;
        pmask_out = ~0ull;
        return;
    }
    int hi = 63 - __clzll(diff);
    uint64_t pmask = (hi == 63) ? 0ull : (~0ull << (hi + 1));
    uint64_t prefix = mx & pmask;
    uint32_t need = kk;
    for (;;) {
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
        hi = shift - 1;
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

// Descending bitonic sort of s[0..n), n a power of two <= NT: one element per
// thread, partners closer than 64 exchanged with lane shuffles, farther ones
// through LDS.  Callers barrier before; ends with a barrier.
template <int NT>
__device__ void bitonic_desc_reg(uint64_t *s, int n) {
    const int i = threadIdx.x;
    uint64_t v = (i < n) ? s[i] : 0ull;
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            uint64_t o;
            if (j >= 64) {
                __syncthreads();
                if (i < n) s[i] = v;
                __syncthreads();
                o = (i < n) ? s[i ^ j] : 0ull;
            } else {
                o = shx64(v, j);
            }
            const bool desc = (i & k) == 0;
            const bool lower = (i & j) == 0;
            const uint64_t mx = v > o ? v : o, mn = v > o ? o : v;
            v = (desc == lower) ? mx : mn;
        }
    }
    __syncthreads();
    if (i < n) s[i] = v;
    __syncthreads();
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
    const int64_t i0 = P.offsets[b], i1 = P.offsets[b + 1];
    for (int64_t t = i0 + threadIdx.x; t < i1; t += NT) {
        int64_t r = (int64_t)P.ids[t] - seg0;
        if (r >= 0 && r < len) atomicOr(&bm[r >> 5], 1u << (r & 31));
    }
    __syncthreads();
}

__device__ __forceinline__ const void *row_ptr(const KParams &P, int dt, int b) {
    return (const char *)P.logits + (int64_t)b * P.ld * (dt == 1 ? 2 : 4);
}

// ================================================================== chunk passes

constexpr int U = 4;           // k_stream: tiles per batch (256 threads)
constexpr int SEL_THREADS = 512;
constexpr int SEL_DEPTH = 4;   // k_select: batches in flight

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

// Issue the loads of one batch (UU groups per thread; row-relative offsets).
template <int DT, bool AL, int NT, int UU>
__device__ __forceinline__ void issue_batch(const void *rowp, int base, int c1,
                                            Raw<DT> (&raw)[UU]) {
#pragma unroll
    for (int u = 0; u < UU; ++u) {
        const int j = base + (u * NT + (int)threadIdx.x) * VEC;
        load_raw<DT, AL>(rowp, j, group_nv(j, c1), raw[u]);
    }
}

// Widen and transform a loaded batch.  FULL: the whole batch lies inside the
// chunk (no per-element bounds).
template <int DT, int NT, int UU, bool XF, bool FULL, bool CANON = true>
__device__ __forceinline__ void finish_batch(const Raw<DT> (&raw)[UU], int base, int c0, int c1,
                                             const uint32_t *bm, const KParams &P,
                                             float (&x)[UU][8], int (&jb)[UU], int (&nv)[UU]) {
#pragma unroll
    for (int u = 0; u < UU; ++u) {
        jb[u] = base + (u * NT + (int)threadIdx.x) * VEC;
        nv[u] = FULL ? 8 : group_nv(jb[u], c1);
        unpack_raw<DT>(raw[u], x[u]);
        const uint32_t bits = (FULL || nv[u] > 0) ? pen_bits<XF>(bm, jb[u] - c0, P) : 0u;
        if (XF || CANON) {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[u][i] = xform<XF>(x[u][i], (bits >> i) & 1u, P);
        }
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
template <int UU>
__device__ __forceinline__ void stats_batch(Stats &st, const float (&x)[UU][8], const int (&nv)[UU]) {
    float tm = -INFINITY;
#pragma unroll
    for (int u = 0; u < UU; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i)
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
            for (int i = 0; i < 8; ++i)
                if (i < nv[u]) zs += __expf(x[u][i] - st.m);
            st.z += (double)zs;
        }
    }
}

// Workgroup merge of per-thread Stats into one ChunkStat's m / z / xmin.
template <int NT>
__device__ __forceinline__ void stats_reduce(const Stats &st, float *scf, double *scd, ChunkStat &cs) {
    float m = st.m;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, shxf(m, s));
    if ((threadIdx.x & 63) == 0) scf[threadIdx.x >> 6] = m;
    __syncthreads();
    float M = scf[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) M = fmaxf(M, scf[i]);
    __syncthreads();
    double z = (st.z != 0.0) ? st.z * exp((double)st.m - (double)M) : 0.0;
    z = wg_sum_f64<NT>(z, scd);
    float mn = st.xmin;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) mn = fminf(mn, shxf(mn, s));
    if ((threadIdx.x & 63) == 0) scf[threadIdx.x >> 6] = mn;
    __syncthreads();
    float MN = scf[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) MN = fminf(MN, scf[i]);
    __syncthreads();
    cs.m = M;
    cs.z = z;
    cs.xmin = MN;
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

// ---------------------------------------------------------------- k_stream
// Rows with neither top-k nor top-p: K is the whole row.  Writes the dense
// output (x itself), runs the exponential race over the whole chunk (q is
// streamed in the same pass) or the greedy argmax, and (for the optional
// probabilities) the chunk's max / sum-exp.  No barrier in the loop.
// For rows with top-k or top-p the first workgroup of the row estimates the
// admission value the select pass filters with.

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
// their distance below the sample maximum, first in steps of 2^16 (one bf16
// ulp), and in steps of 2^24 when the 255 top bins hold fewer than r; only
// the top 255 bins are counted, so the bins stay sparse and the LDS atomics
// rarely collide.  -inf (admit everything) when r would exceed the sample.
// Only the speed of the select pass depends on t: that pass checks that what
// it admitted holds the row's kk largest and redoes the row exactly when it
// does not.
// First element of sample run s of row b (V > EST_N): inside the s-th of
// EST_SEGS equal segments, at one of 16 offsets that depend on s and b, a
// multiple of 8.  Staggered so that the runs of all rows do not start at
// the same offsets modulo a large power of two, where they would all fall
// on the same few memory channels.
__device__ __forceinline__ int est_run_start(int s, int b, int V) {
    const int64_t seg0 = ((int64_t)s * V / EST_SEGS) & ~(int64_t)(VEC - 1);
    const int64_t seg1 = ((int64_t)(s + 1) * V / EST_SEGS) & ~(int64_t)(VEC - 1);
    const int64_t room = seg1 - seg0 - EST_SEG;  // >= 0 when V > EST_N
    const int64_t step = (room / 16) & ~(int64_t)(VEC - 1);
    return (int)(seg0 + (int64_t)((s * 5 + b * 3) & 15) * step);
}

template <int DT, bool AL>
__device__ __forceinline__ float row_estimate(const KParams &P, int b, uint32_t kk, StreamShared &S) {
    constexpr int NT = K1_THREADS;
    constexpr int PER = EST_N / (NT * VEC);  // groups of 8 per thread
    constexpr int GPS = EST_SEG / VEC;       // groups per run
    const int V = P.V;
    const bool whole = V <= EST_N;
    const int n = whole ? V : EST_N;
    const double r0 = (double)kk * (double)n / (double)V;
    const double rr = ceil(r0 + 4.0 * sqrt(r0) + 8.0);
    if (rr >= (double)n) return -INFINITY;
    const uint32_t r = (uint32_t)rr;
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
    // the sample maximum
    uint32_t mx = 0;
#pragma unroll
    for (int g = 0; g < PER; ++g) {
        float x[8];
        unpack_raw<DT>(raw[g], x);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < nv[g]) mx = max(mx, f2key(x[i]));
    }
#pragma unroll
    for (int sft = 32; sft >= 1; sft >>= 1) mx = max(mx, shx(mx, sft));
    if ((threadIdx.x & 63) == 0) S.sci[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = S.sci[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) mx = max(mx, S.sci[i]);
    for (int shift = 16; shift <= 24; shift += 8) {
        for (int i = threadIdx.x; i < 256; i += NT) S.hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int g = 0; g < PER; ++g) {
            float x[8];
            unpack_raw<DT>(raw[g], x);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t d = (mx - f2key(x[i])) >> shift;
                if (i < nv[g] && d < 255u) atomicAdd(&S.hist[255 - d], 1u);
            }
        }
        __syncthreads();
        uint32_t tot = 0;
        if (threadIdx.x < 64) {
            tot = S.hist[4 * threadIdx.x] + S.hist[4 * threadIdx.x + 1] +
                  S.hist[4 * threadIdx.x + 2] + S.hist[4 * threadIdx.x + 3];
#pragma unroll
            for (int sft = 32; sft >= 1; sft >>= 1) tot += shx(tot, sft);
            if (threadIdx.x == 0) S.sel[3] = tot;
        }
        __syncthreads();
        tot = S.sel[3];
        if (tot >= r || shift == 24) {
            if (tot < r) return -INFINITY;  // unreachable: 255 * 2^24 spans every key
            wave0_find_bin(S.hist, r, S.sel);
            __syncthreads();
            const uint32_t d = 255u - S.sel[0];
            // every key of bins 0..d, i.e. key > mx - (d + 1) * 2^shift
            const uint64_t lo = (uint64_t)mx - (((uint64_t)d + 1) << shift) + 1;
            const uint32_t fk = lo > (uint64_t)mx ? 0u : (uint32_t)lo;
            return fk <= f2key(-INFINITY) ? -INFINITY : key2f(fk);
        }
        __syncthreads();
    }
    return -INFINITY;
}

struct StreamState {
    Stats st;
    Race rc;
    uint64_t am;
};

template <int DT, bool AL, bool XF, bool FULL>
__device__ __forceinline__ void stream_batch(const Raw<DT> (&cur)[U], int base, int c0, int c1,
                                             const uint32_t *bm, const KParams &P, float *rowo,
                                             const float *rowq, bool do_stats, bool do_race,
                                             StreamState &ss) {
    float x[U][8];
    int jb[U], nv[U];
    finish_batch<DT, K1_THREADS, U, XF, FULL>(cur, base, c0, c1, bm, P, x, jb, nv);
    if (rowo) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (FULL || nv[u] > 0) store8<AL>(rowo, jb[u], nv[u], x[u]);
    }
    if (do_stats) stats_batch(ss.st, x, nv);
    if (do_race) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float qv[8];
            load8<0, AL>(rowq, jb[u], nv[u], qv);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (FULL || i < nv[u]) race_offer(ss.rc, x[u][i], qv[i] + P.eps, (uint32_t)(jb[u] + i));
        }
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (FULL || i < nv[u]) {
                    const uint64_t cv = mkcomp(x[u][i], (uint32_t)(jb[u] + i));
                    ss.am = cv > ss.am ? cv : ss.am;
                }
    }
}

template <int DT, bool AL, bool XF>
__global__ __launch_bounds__(K1_THREADS) void k_stream(KParams P, KPlan L, KWork W) {
    __shared__ StreamShared S;
    extern __shared__ uint32_t bm[];  // penalty bitmap of the chunk
    const int tid = threadIdx.x;
    const int b = blockIdx.x / L.nch, c = blockIdx.x % L.nch;
    if (c == 0 && tid == 0) {
        W.rowkey[b] = 0u;  // the row's exact admission key
        W.rmask[b] = 0u;   // no chunk redone
    }
    const Mode md = row_mode(P, b);
    if (md.tk || md.tp) {
        // one workgroup per row estimates; which one rotates with the row so
        // the estimates spread over the XCDs (workgroup i runs on XCD i % 8)
        if (c == b % L.nch) {
            const uint32_t kk = md.tk ? (uint32_t)md.k : (uint32_t)min(P.guess, P.V);
            const float t = row_estimate<DT, AL>(P, b, kk, S);
            if (tid == 0) W.rowthr[b] = t;
        }
        return;
    }
    const int c0 = c * (int)L.chunk_len;
    const int c1 = min(c0 + (int)L.chunk_len, P.V);
    const int slot = b * NCH_MAX + c;
    if (c0 >= c1) {
        if (tid == 0) {
            W.ccnt[slot] = 0;
            W.cstat[slot] = empty_stat();
        }
        return;
    }
    if (XF && P.pen) build_bitmap<K1_THREADS>(bm, c0, c1 - c0, P, b);
    const bool do_race = md.sm;
    const bool do_stats = (P.flags & NEED_PROBS) != 0;
    const void *rowp = row_ptr(P, DT, b);
    const float *rowq = P.q ? P.q + (int64_t)b * P.V : nullptr;
    float *rowo = P.out_logits ? P.out_logits + (int64_t)b * P.V : nullptr;

    StreamState ss;
    ss.st.m = -INFINITY; ss.st.xmin = INFINITY; ss.st.z = 0.0;
    ss.rc.x = -INFINITY; ss.rc.qe = 1.0f; ss.rc.idx = NONE;
    ss.am = 0;
    constexpr int BATCH = K1_THREADS * VEC * U;
    Raw<DT> cur[U], nxt[U];
    issue_batch<DT, AL, K1_THREADS, U>(rowp, c0, c1, cur);
    for (int base = c0; base < c1; base += BATCH) {
        if (base + BATCH < c1) issue_batch<DT, AL, K1_THREADS, U>(rowp, base + BATCH, c1, nxt);
        if (base + BATCH <= c1)
            stream_batch<DT, AL, XF, true>(cur, base, c0, c1, bm, P, rowo, rowq, do_stats, do_race, ss);
        else
            stream_batch<DT, AL, XF, false>(cur, base, c0, c1, bm, P, rowo, rowq, do_stats, do_race, ss);
#pragma unroll
        for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    }
    ChunkStat cs = empty_stat();
    if (do_stats) stats_reduce<K1_THREADS>(ss.st, S.scx, S.scd, cs);
    if (do_race) {
        Race r = wg_race<K1_THREADS>(ss.rc, S.scx, S.scq, S.sci);
        cs.rx = r.x;
        cs.rqe = r.qe;
        cs.ridx = r.idx;
    } else {
        const uint64_t am = wg_max_u64<K1_THREADS>(ss.am, S.sc64);
        if (tid == 0) {
            W.cand[(int64_t)slot * SLOT] = am;
            W.ccnt[slot] = 1;
        }
    }
    if (tid == 0) W.cstat[slot] = cs;
}

// ---------------------------------------------------------------- k_select
// Rows with top-k and/or top-p.  Keeps a superset of the chunk's kk largest
// (kk = k, or the top-k guess G for top-p rows without top-k) in an LDS
// buffer: an element enters when its value key is >= the admission key; when
// the buffer fills it is cut back to a superset of its kk largest -- with a
// 256-bin value histogram (the kept part is every entry at or above the bin
// where the count from the top reaches kk), or an exact radix select when
// one bin holds too many equal or near-equal values -- and the admission key
// becomes the smallest kept value.  This is the rolling, prefiltered top-k of
// the Ascend npu_top_k_top_p_sample page (topK section) with the exact cut
// deferred to the row merge.  Top-p rows without top-k also accumulate the
// chunk's max / sum-exp for the softmax over the whole row.

struct SelShared {
    uint64_t buf[2][SEL_CAP];  // candidate buffer, two halves used in turn
    uint32_t hist[256];
    uint32_t sel[4];
    uint32_t sc[16];
    uint64_t sc64[16];
    double scd[16];
    float scf[16];
    uint32_t cnt;    // reserved entries of the active half
    uint32_t ffail;  // first reservation that did not fit
    uint32_t kcnt;   // entries written by a compaction
    uint32_t rkey;   // admission key published by the row's other chunks
    float shi[SEL_THREADS / 64];  // per-wave largest appended value
};

__device__ __forceinline__ uint32_t bin256(float x, float lo, float scale) {
    float t = (x - lo) * scale;
    if (!(t >= 0.0f)) return 0u;
    if (t >= 255.0f) return 255u;
    return (uint32_t)t;
}

__device__ __forceinline__ uint32_t lane_rank(uint64_t bal) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

// Workgroup reduction of (count, finite min, max) over SEL_THREADS threads.
__device__ __forceinline__ void sel_span(SelShared &S, uint32_t &cnt, float &lo, float &hi) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        cnt += shx(cnt, s);
        lo = fminf(lo, shxf(lo, s));
        hi = fmaxf(hi, shxf(hi, s));
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        S.sc[w] = cnt;
        S.scf[w] = lo;
        S.scf[8 + w] = hi;
    }
    __syncthreads();
    cnt = S.sc[0];
    lo = S.scf[0];
    hi = S.scf[8];
#pragma unroll
    for (int i = 1; i < SEL_THREADS / 64; ++i) {
        cnt += S.sc[i];
        lo = fminf(lo, S.scf[i]);
        hi = fmaxf(hi, S.scf[8 + i]);
    }
    __syncthreads();
}

// Exact radix select over the entries of src[0..n) whose value key is >=
// tkey (distinct composites, 1 <= kk < their count), read from LDS in every
// pass: (v & pmask) >= prefix holds for exactly the kk largest of them.
// Common high bits are skipped first.
template <int NT>
__device__ void radix_select_lds(const uint64_t *src, uint32_t n, uint32_t tkey, uint32_t kk,
                                 SelShared &S, uint64_t &prefix_out, uint64_t &pmask_out) {
    uint64_t mn = ~0ull, mx = 0ull;
    for (uint32_t i = threadIdx.x; i < n; i += NT) {
        const uint64_t v = src[i];
        if ((uint32_t)(v >> 32) >= tkey) {
            mn = v < mn ? v : mn;
            mx = v > mx ? v : mx;
        }
    }
    mn = wg_min_u64<NT>(mn, S.sc64);
    mx = wg_max_u64<NT>(mx, S.sc64);
    const uint64_t diff = mn ^ mx;
    if (diff == 0) {
        prefix_out = mx;
        pmask_out = ~0ull;
        return;
    }
    int hi = 63 - __clzll(diff);
    uint64_t pmask = (hi == 63) ? 0ull : (~0ull << (hi + 1));
    uint64_t prefix = mx & pmask;
    uint32_t need = kk;
    for (;;) {
        const int width = hi + 1 < 8 ? hi + 1 : 8;
        const int shift = hi + 1 - width;
        const uint32_t dmask = (1u << width) - 1u;
        for (int i = threadIdx.x; i < 256; i += NT) S.hist[i] = 0;
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < n; i += NT) {
            const uint64_t v = src[i];
            if ((uint32_t)(v >> 32) >= tkey && (v & pmask) == prefix)
                atomicAdd(&S.hist[(uint32_t)(v >> shift) & dmask], 1u);
        }
        __syncthreads();
        wave0_find_bin(S.hist, need, S.sel);
        __syncthreads();
        const uint32_t d = S.sel[0], above = S.sel[1], cntd = S.sel[2];
        need -= above;
        prefix |= (uint64_t)d << shift;
        pmask |= (uint64_t)dmask << shift;
        if (cntd == need || shift == 0) break;
        hi = shift - 1;
    }
    prefix_out = prefix;
    pmask_out = pmask;
}

// Cut S.buf[half][0..n) (n > kk) back to a superset of the kk largest of its
// entries whose value key is >= tkey, holding at most `limit` entries (limit
// >= kk): every such entry at or above the 256-bin value-histogram bin where
// the count from the top reaches kk -- bins span [value(tkey), hi], hi an
// upper bound of the buffer -- or exactly the kk largest when that bin is too
// full.  The survivors go to the other half.  Returns their count; when at
// least kk survive, tkey rises to the smallest surviving key.
__device__ uint32_t sel_reduce(SelShared &S, int half, uint32_t n, uint32_t kk, uint32_t limit,
                               uint32_t &tkey, float hi) {
    constexpr int NT = SEL_THREADS;
    const uint64_t *src = S.buf[half];
    uint64_t *dst = S.buf[half ^ 1];
    float lo = key2f(tkey);
    if (tkey == 0u) {
        // no floor yet: take the smallest finite value in the buffer
        lo = INFINITY;
        for (uint32_t i = threadIdx.x; i < n; i += NT) {
            const float xv = cval(src[i]);
            if (xv > -INFINITY) lo = fminf(lo, xv);
        }
        uint32_t dummy = 0;
        float dh = -INFINITY;
        sel_span(S, dummy, lo, dh);
    }
    if (threadIdx.x == 0) S.kcnt = 0;
    bool exact = true;
    uint32_t bstar = 0;
    float scale = 0.0f;
    if (hi > lo && lo > -INFINITY) {
        scale = 256.0f / (hi - lo);
        for (int i = threadIdx.x; i < 256; i += NT) S.hist[i] = 0;
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < n; i += NT) {
            const uint64_t v = src[i];
            if ((uint32_t)(v >> 32) >= tkey) atomicAdd(&S.hist[bin256(cval(v), lo, scale)], 1u);
        }
        __syncthreads();
        // fewer than kk entries at or above the floor: keep them all
        uint32_t tot = 0;
        if (threadIdx.x < 64) {
            const uint32_t t4 = S.hist[4 * threadIdx.x] + S.hist[4 * threadIdx.x + 1] +
                                S.hist[4 * threadIdx.x + 2] + S.hist[4 * threadIdx.x + 3];
            tot = t4;
#pragma unroll
            for (int sft = 32; sft >= 1; sft >>= 1) tot += shx(tot, sft);
            if (threadIdx.x == 0) S.sel[3] = tot;
        }
        __syncthreads();
        tot = S.sel[3];
        if (tot <= kk) {
            bstar = 0;
            exact = false;
        } else {
            wave0_find_bin(S.hist, kk, S.sel);
            __syncthreads();
            bstar = S.sel[0];
            exact = S.sel[1] + S.sel[2] > limit;
        }
    }
    uint64_t prefix = 0, pmask = 0;
    if (exact) {
        uint32_t cnt = 0;
        for (uint32_t i = threadIdx.x; i < n; i += NT) cnt += (uint32_t)(src[i] >> 32) >= tkey;
        float l2 = 0.0f, h2 = 0.0f;
        sel_span(S, cnt, l2, h2);
        if (cnt > kk) {
            radix_select_lds<NT>(src, n, tkey, kk, S, prefix, pmask);
        } else {
            exact = false;  // keep every entry at or above the floor
            bstar = 0;
            scale = 0.0f;
            lo = 0.0f;
        }
    }
    const int lane = threadIdx.x & 63;
    uint32_t mk = NONE;
    const uint32_t rounds = (n + NT - 1) / NT;
    for (uint32_t rd = 0; rd < rounds; ++rd) {
        const uint32_t i = rd * NT + threadIdx.x;
        const uint64_t v = (i < n) ? src[i] : 0ull;
        bool keep = i < n && (uint32_t)(v >> 32) >= tkey;
        if (keep) keep = exact ? ((v & pmask) >= prefix) : (bin256(cval(v), lo, scale) >= bstar);
        const uint64_t bal = __ballot(keep);
        if (bal == 0) continue;
        uint32_t wbase = 0;
        if (lane == 0) wbase = atomicAdd(&S.kcnt, (uint32_t)__popcll(bal));
        wbase = (uint32_t)__shfl((int)wbase, 0, 64);
        if (keep) {
            dst[wbase + lane_rank(bal)] = v;
            const uint32_t k = (uint32_t)(v >> 32);
            mk = k < mk ? k : mk;
        }
    }
    mk = wg_min_u32<NT>(mk, S.sc);
    const uint32_t kept = S.kcnt;
    if (kept >= kk && mk != NONE && mk > tkey) tkey = mk;
    return kept;
}

// Append the elements of one group of 8 (values x[], first id j, nv valid)
// with x >= tval to the active half: one LDS reservation per wave, slots
// placed with ballots; hi tracks the largest value appended.  Returns true
// when the wave's reservation did not fit (nothing written; the group stays
// pending).
template <bool FULL>
__device__ __forceinline__ bool sel_append(SelShared &S, int half, const float (&x)[8], uint32_t j,
                                           int nv, float tval, float &hi) {
    const int lane = threadIdx.x & 63;
    uint64_t bal[8];
    uint32_t tot = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        bal[i] = __ballot((FULL || i < nv) && x[i] >= tval);
        tot += (uint32_t)__popcll(bal[i]);
    }
    if (tot == 0) return false;
    uint32_t wbase = 0;
    if (lane == 0) wbase = atomicAdd(&S.cnt, tot);
    wbase = (uint32_t)__shfl((int)wbase, 0, 64);
    if (wbase + tot > (uint32_t)SEL_CAP) {
        if (lane == 0) atomicMin(&S.ffail, wbase);
        return true;
    }
    uint64_t *dst = S.buf[half];
    uint32_t off = wbase;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (bal[i] == 0) continue;
        if ((bal[i] >> lane) & 1ull) {
            const float xc = x[i] + 0.0f;  // -0 -> +0 before the key
            dst[off + lane_rank(bal[i])] = mkcomp(xc, j + i);
            hi = fmaxf(hi, xc);
        }
        off += (uint32_t)__popcll(bal[i]);
    }
    return false;
}

__device__ __forceinline__ float key_floor(uint32_t tkey) {
    return tkey ? key2f(tkey) : -INFINITY;
}

// Admission key from one group of 8 per thread held in registers (the first
// batch of a chunk): a value key k such that at least kk of the batch's
// elements have key >= k, taken at the 256-bin histogram bin where the
// count from the top reaches kk.  0 (admit everything) when the batch has
// fewer than kk elements.
__device__ uint32_t batch_key(SelShared &S, const float (&x)[8], int nv, uint32_t kk) {
    uint32_t cnt = 0;
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i < nv) {
            ++cnt;
            if (x[i] > -INFINITY) {
                lo = fminf(lo, x[i]);
                hi = fmaxf(hi, x[i]);
            }
        }
    sel_span(S, cnt, lo, hi);
    if (cnt < kk || !(hi > lo)) return 0u;
    const float scale = 256.0f / (hi - lo);
    for (int i = threadIdx.x; i < 256; i += SEL_THREADS) S.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i < nv) atomicAdd(&S.hist[bin256(x[i], lo, scale)], 1u);
    __syncthreads();
    wave0_find_bin(S.hist, kk, S.sel);
    __syncthreads();
    const uint32_t bstar = S.sel[0];
    uint32_t mk = NONE;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i < nv && bin256(x[i], lo, scale) >= bstar) mk = min(mk, f2key(x[i] + 0.0f));
    mk = wg_min_u32<SEL_THREADS>(mk, S.sc);
    return mk == NONE ? 0u : mk;
}

// One batch before the workgroup barrier: widen/transform, top-p statistics,
// the first batch's admission key, and the append.  Returns true when this
// wave's append did not fit.
template <int DT, bool XF, bool FULL>
__device__ __forceinline__ bool select_front(SelShared &S, const Raw<DT> &cur, int base, int c0,
                                             int c1, const uint32_t *bm, const KParams &P,
                                             bool do_stats, Stats &st, bool &first, uint32_t kk,
                                             uint32_t &tkey, uint32_t &rk_seen, uint32_t *rowkey,
                                             int half, float &hi, float (&xo)[8], int &j0,
                                             int &nv0) {
    float x[1][8];
    int jb[1], nv[1];
    finish_batch<DT, SEL_THREADS, 1, XF, FULL, false>(*(const Raw<DT>(*)[1]) & cur, base, c0, c1,
                                                      bm, P, x, jb, nv);
    if (do_stats) stats_batch(st, x, nv);
    if (first) {
        // the first batch sets the admission key from its own values
        first = false;
        tkey = batch_key(S, x[0], nv[0], kk);
        if (threadIdx.x == 0 && tkey) rk_seen = atomicMax(rowkey, tkey);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) xo[i] = x[0][i];
    j0 = jb[0];
    nv0 = nv[0];
    return sel_append<FULL>(S, half, x[0], (uint32_t)j0, nv0, key_floor(tkey), hi);
}

// Exact selection over the chunk [c0, c1) of row b, appended to the `valid`
// entries already in S.buf[half] (hi: an upper bound of their values, or
// -inf): on return S.buf[half] holds `valid` entries, and every element of
// the chunk and of the earlier entries that is among their kk largest, or
// whose value key is >= the returned tkey (tkey only rises), is among them.
// tkey on entry is a valid admission key for the row (0 = none).  The
// penalty bitmap bm must describe [c0, c1).
template <int DT, bool AL, bool XF>
__device__ void select_exact(SelShared &S, const KParams &P, const uint32_t *bm,
                             const void *rowp, int c0, int c1, uint32_t kk, bool do_stats,
                             Stats &st, uint32_t *rowkey, uint32_t &tkey, int &half,
                             uint32_t &valid, float &hi) {
    const int tid = threadIdx.x;
    if (tid == 0) {
        S.cnt = valid;
        S.ffail = NONE;
    }
    __syncthreads();
    uint32_t rk_seen = 0;  // thread 0: row key returned by the last publication
    bool first = true;
    constexpr int BATCH = SEL_THREADS * VEC;
    Raw<DT> ring[SEL_DEPTH];
#pragma unroll
    for (int d = 0; d < SEL_DEPTH; ++d)
        if (c0 + d * BATCH < c1)
            issue_batch<DT, AL, SEL_THREADS, 1>(rowp, c0 + d * BATCH, c1, *(Raw<DT>(*)[1]) & ring[d]);
    for (int base = c0; base < c1; base += BATCH) {
        const Raw<DT> cur = ring[0];
#pragma unroll
        for (int d = 0; d + 1 < SEL_DEPTH; ++d) ring[d] = ring[d + 1];
        if (base + SEL_DEPTH * BATCH < c1)
            issue_batch<DT, AL, SEL_THREADS, 1>(rowp, base + SEL_DEPTH * BATCH, c1,
                                               *(Raw<DT>(*)[1]) & ring[SEL_DEPTH - 1]);
        float x[8];
        int j0, nv0;
        const uint32_t tk_in = tkey;
        bool pending =
            (base + BATCH <= c1)
                ? select_front<DT, XF, true>(S, cur, base, c0, c1, bm, P, do_stats, st, first, kk,
                                             tkey, rk_seen, rowkey, half, hi, x, j0, nv0)
                : select_front<DT, XF, false>(S, cur, base, c0, c1, bm, P, do_stats, st, first, kk,
                                              tkey, rk_seen, rowkey, half, hi, x, j0, nv0);
        tkey = max(tkey, tk_in);
        __syncthreads();
        uint32_t ff = S.ffail;
        valid = min(S.cnt, ff);
        bool ovf = ff != NONE;
        while (ovf || valid > (uint32_t)SEL_SOFT) {
            // adopt the key the row's other chunks have published, cut back
            float h = hi;
#pragma unroll
            for (int sft = 32; sft >= 1; sft >>= 1) h = fmaxf(h, shxf(h, sft));
            if ((tid & 63) == 0) S.shi[tid >> 6] = h;
            if (tid == 0) S.rkey = rk_seen;
            __syncthreads();
            tkey = max(tkey, S.rkey);
            h = S.shi[0];
#pragma unroll
            for (int i = 1; i < SEL_THREADS / 64; ++i) h = fmaxf(h, S.shi[i]);
            const uint32_t kept = sel_reduce(S, half, valid, kk, SEL_LIMIT, tkey, h);
            half ^= 1;
            if (tid == 0) {
                S.cnt = kept;
                S.ffail = NONE;
                rk_seen = atomicMax(rowkey, tkey);
            }
            __syncthreads();
            valid = kept;
            if (!ovf) break;
            if (pending) pending = sel_append<false>(S, half, x, (uint32_t)j0, nv0, key_floor(tkey), hi);
            __syncthreads();
            ff = S.ffail;
            valid = min(S.cnt, ff);
            ovf = ff != NONE;
        }
    }
    // the latest row key bounds every chunk's output
    if (tid == 0)
        S.rkey = max(rk_seen,
                     (uint32_t)__hip_atomic_load(rowkey, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    __syncthreads();
    tkey = max(tkey, S.rkey);
    __syncthreads();
}

// ---------------------------------------------------------------- k_select
// Fast pass over one chunk of a top-k / top-p row: one streaming pass, no
// barrier, admitting against the row's estimated value (see row_estimate).
// A chunk whose admissions do not fit the buffer hands over nothing and is
// marked (count -1) for the exact pass; so is, in effect, a row whose fast
// chunks turn out not to hold its kk largest (k_fix decides).

struct FastShared {
    uint64_t buf[SLOT];  // admitted entries
    uint32_t cnt;        // reserved entries
    uint32_t ffail;      // set when a reservation did not fit
    uint32_t nstr;       // admitted entries with y > yt
    float scf[16];
    double scd[16];
};

// Admit the elements of one group of 8 (first id j): non-penalised elements
// with raw x >= traw, penalised ones (and, for rows that accumulate
// statistics, all of them) with transformed y >= yt, where yt is the
// transform of traw; every element left out therefore has y <= yt.  One LDS
// reservation per wave; a reservation that does not fit sets S.ffail and
// writes nothing.
template <int DT, bool XF, bool FULL>
__device__ __forceinline__ void fast_group(FastShared &S, const Raw<DT> &cur, int j, int c0,
                                           int c1, const uint32_t *bm, const KParams &P,
                                           bool do_stats, Stats &st, float traw, float yt) {
    const int lane = threadIdx.x & 63;
    const int nv = FULL ? 8 : group_nv(j, c1);
    float x[8];
    unpack_raw<DT>(cur, x);
    const uint32_t bits = (FULL || nv > 0) ? pen_bits<XF>(bm, j - c0, P) : 0u;
    bool pass[8];
    if (do_stats) {
        float y[1][8];
        int nvv[1] = {nv};
#pragma unroll
        for (int i = 0; i < 8; ++i) y[0][i] = xform<XF>(x[i], (bits >> i) & 1u, P);
        stats_batch(st, y, nvv);
#pragma unroll
        for (int i = 0; i < 8; ++i) pass[i] = (FULL || i < nv) && y[0][i] >= yt;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) pass[i] = (FULL || i < nv) && x[i] >= traw;
        if (XF && bits) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if ((bits >> i) & 1u) pass[i] = (FULL || i < nv) && xform<XF>(x[i], 1u, P) >= yt;
        }
    }
    uint64_t bal[8];
    uint32_t tot = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        bal[i] = __ballot(pass[i]);
        tot += (uint32_t)__popcll(bal[i]);
    }
    if (tot == 0) return;
    uint32_t wbase = 0;
    if (lane == 0) wbase = atomicAdd(&S.cnt, tot);
    wbase = (uint32_t)__shfl((int)wbase, 0, 64);
    if (wbase + tot > (uint32_t)SLOT) {
        if (lane == 0) S.ffail = 1u;
        return;
    }
    uint32_t off = wbase;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (bal[i] == 0) continue;
        if (pass[i]) {
            const float y = xform<XF>(x[i], (bits >> i) & 1u, P);
            S.buf[off + lane_rank(bal[i])] = mkcomp(y, (uint32_t)(j + i));
        }
        off += (uint32_t)__popcll(bal[i]);
    }
}

// Batches in flight per thread: 8 groups of bf16 or 4 of fp32 (128 bytes).
template <int DT>
struct FastDepth {
    static constexpr int value = DT == 1 ? 8 : 4;
};

template <int DT, bool AL, bool XF>
__global__ __launch_bounds__(SEL_THREADS, 8) void k_select(KParams P, KPlan L, KWork W) {
    __shared__ FastShared S;
    extern __shared__ uint32_t bm[];  // penalty bitmap of the chunk
    const int tid = threadIdx.x;
    const int b = blockIdx.x / L.nch, c = blockIdx.x % L.nch;
    const Mode md = row_mode(P, b);
    if (!(md.tk || md.tp)) return;
    // every one of the L.nch chunks of a row is non-empty
    const int c0 = c * (int)L.chunk_len;
    const int c1 = min(c0 + (int)L.chunk_len, P.V);
    const int slot = b * NCH_MAX + c;
    const bool do_stats = !md.tk;
    const void *rowp = row_ptr(P, DT, b);
    const float traw = W.rowthr[b];
    const float yt = xform<XF>(traw, 0u, P);
    if (XF && P.pen) build_bitmap<SEL_THREADS>(bm, c0, c1 - c0, P, b);
    if (tid == 0) {
        S.cnt = 0;
        S.ffail = 0;
        S.nstr = 0;
    }
    __syncthreads();

    Stats st;
    st.m = -INFINITY; st.xmin = INFINITY; st.z = 0.0;
    constexpr int D = FastDepth<DT>::value;
    constexpr int BATCH = SEL_THREADS * VEC;
    const int jt = tid * VEC;
    Raw<DT> ring[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const int j = c0 + d * BATCH + jt;
        if (c0 + d * BATCH < c1) load_raw<DT, AL>(rowp, j, group_nv(j, c1), ring[d]);
    }
    for (int base = c0; base < c1; base += D * BATCH) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int bb = base + d * BATCH;
            if (bb < c1) {
                if (bb + BATCH <= c1)
                    fast_group<DT, XF, true>(S, ring[d], bb + jt, c0, c1, bm, P, do_stats, st, traw, yt);
                else
                    fast_group<DT, XF, false>(S, ring[d], bb + jt, c0, c1, bm, P, do_stats, st, traw, yt);
                const int nb = bb + D * BATCH;
                if (nb < c1) load_raw<DT, AL>(rowp, nb + jt, group_nv(nb + jt, c1), ring[d]);
            }
        }
    }
    __syncthreads();
    const bool ovf = S.ffail != 0u;
    const uint32_t n = S.cnt;
    if (!ovf) {
        // hand the admitted entries over as they are, counting those above yt
        uint64_t *dst = W.cand + (int64_t)slot * SLOT;
        uint32_t strict = 0;
        for (uint32_t i = tid; i < n; i += SEL_THREADS) {
            const uint64_t v = S.buf[i];
            dst[i] = v;
            strict += cval(v) > yt;
        }
#pragma unroll
        for (int sft = 32; sft >= 1; sft >>= 1) strict += shx(strict, sft);
        if ((tid & 63) == 0 && strict) atomicAdd(&S.nstr, strict);
    }
    ChunkStat cs = empty_stat();
    if (do_stats) stats_reduce<SEL_THREADS>(st, S.scf, S.scd, cs);
    __syncthreads();
    if (tid == 0) {
        cs.nstr = S.nstr;
        W.ccnt[slot] = ovf ? -1 : (int32_t)n;
        W.cstat[slot] = cs;
    }
}

// ---------------------------------------------------------------- k_fix
// Exact selection, one workgroup per top-k / top-p row, for what the fast
// pass could not settle: chunks that overflowed, and -- when fewer than kk
// of the entries handed over lie above the row's estimated value yt, so the
// row's kk-th largest may be an element a fast chunk left out (those all
// have y <= yt) -- the fast chunks too.  Everything it selects goes to the
// row's redo slot, which replaces the chunks in rmask.

// Copy the entries of S.buf[half][0..n) whose value key is >= tkey to dst;
// their number ends in S.kcnt.
__device__ void copy_out(SelShared &S, int half, uint32_t n, uint32_t tkey, uint64_t *dst) {
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid == 0) S.kcnt = 0;
    __syncthreads();
    const uint32_t rounds = (n + SEL_THREADS - 1) / SEL_THREADS;
    for (uint32_t rd = 0; rd < rounds; ++rd) {
        const uint32_t i = rd * SEL_THREADS + tid;
        const uint64_t v = (i < n) ? S.buf[half][i] : 0ull;
        const bool keep = i < n && (uint32_t)(v >> 32) >= tkey;
        const uint64_t bal = __ballot(keep);
        if (bal == 0) continue;
        uint32_t wbase = 0;
        if (lane == 0) wbase = atomicAdd(&S.kcnt, (uint32_t)__popcll(bal));
        wbase = (uint32_t)__shfl((int)wbase, 0, 64);
        if (keep) dst[wbase + lane_rank(bal)] = v;
    }
    __syncthreads();
}

// Entries of S.buf[half][0..n) with value key >= tkey and value > yt.
__device__ uint32_t count_above(SelShared &S, int half, uint32_t n, uint32_t tkey, float yt) {
    if (threadIdx.x == 0) S.kcnt = 0;
    __syncthreads();
    uint32_t cnt = 0;
    for (uint32_t i = threadIdx.x; i < n; i += SEL_THREADS) {
        const uint64_t v = S.buf[half][i];
        cnt += (uint32_t)(v >> 32) >= tkey && cval(v) > yt;
    }
#pragma unroll
    for (int sft = 32; sft >= 1; sft >>= 1) cnt += shx(cnt, sft);
    if ((threadIdx.x & 63) == 0 && cnt) atomicAdd(&S.kcnt, cnt);
    __syncthreads();
    const uint32_t tot = S.kcnt;
    __syncthreads();
    return tot;
}

template <int DT, bool AL, bool XF>
__global__ __launch_bounds__(SEL_THREADS, 4) void k_fix(KParams P, KPlan L, KWork W) {
    __shared__ SelShared S;
    extern __shared__ uint32_t bm[];  // penalty bitmap of the chunk being selected
    const int tid = threadIdx.x;
    const int b = xcd_row(blockIdx.x, gridDim.x);
    const Mode md = row_mode(P, b);
    if (!(md.tk || md.tp)) return;
    const int nch = L.nch;
    const int slot0 = b * NCH_MAX;
    uint32_t ovf = 0, fastm = 0, strict = 0;
    for (int c = 0; c < nch; ++c) {
        if (W.ccnt[slot0 + c] < 0) {
            ovf |= 1u << c;
        } else {
            fastm |= 1u << c;
            strict += W.cstat[slot0 + c].nstr;
        }
    }
    const uint32_t kk = md.tk ? (uint32_t)md.k : (uint32_t)min(P.guess, P.V);
    const float traw = W.rowthr[b];
    const float yt = xform<XF>(traw, 0u, P);
    // fast chunks that admitted everything (traw = -inf) are complete
    const bool check = fastm != 0u && traw > -INFINITY;
    if (ovf == 0u && !(check && strict < kk)) return;

    const void *rowp = row_ptr(P, DT, b);
    Stats st;  // unused: the chunk statistics come from the fast pass
    st.m = -INFINITY; st.xmin = INFINITY; st.z = 0.0;
    uint32_t tkey = 0, valid = 0;
    int half = 0;
    float hi = -INFINITY;
    uint32_t jobs = ovf, done = 0;
    for (int phase = 0; phase < 2; ++phase) {
        for (uint32_t m = jobs; m; m &= m - 1) {
            const int cc = __ffs(m) - 1;
            const int d0 = cc * (int)L.chunk_len;
            const int d1 = min(d0 + (int)L.chunk_len, P.V);
            if (XF && P.pen) build_bitmap<SEL_THREADS>(bm, d0, d1 - d0, P, b);
            select_exact<DT, AL, XF>(S, P, bm, rowp, d0, d1, kk, false, st, W.rowkey + b, tkey,
                                     half, valid, hi);
        }
        done |= jobs;
        if (phase > 0 || !check) break;
        if (strict + count_above(S, half, valid, tkey, yt) >= kk) break;
        jobs = fastm;
    }
    copy_out(S, half, valid, tkey, W.rcand + (int64_t)b * SLOT);
    if (tid == 0) {
        W.rcnt[b] = (int32_t)S.kcnt;
        W.rmask[b] = done;
    }
}

// ================================================================== k_rows

struct RowsShared {
    uint64_t srt[KMAX];
    double ev[KMAX];
    double cs[KMAX];
    uint32_t hist[256];
    uint32_t sel[4];
    uint32_t sc[16];
    uint64_t sc64[16];
    double scd[16];
    uint32_t sci[16];
};

template <int NT>
__device__ __forceinline__ uint32_t wg_best_ratio(double r, uint32_t idx, double *scd,
                                                  uint32_t *sci) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        double ro = shxd(r, m);
        uint32_t io = shx(idx, m);
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

__global__ __launch_bounds__(K2_THREADS) void k_rows(KParams P, KPlan L, KWork W) {
    __shared__ RowsShared S;
    const int tid = threadIdx.x;
    const int b = xcd_row(blockIdx.x, gridDim.x);
    const Mode md = row_mode(P, b);
    const bool filtered = md.tk || md.tp;
    const int nch = L.nch;
    const int slot0 = b * NCH_MAX;

    // merged chunk statistics (identical in every thread)
    float M = -INFINITY, XMIN = INFINITY;
    for (int c = 0; c < nch; ++c) {
        M = fmaxf(M, W.cstat[slot0 + c].m);
        XMIN = fminf(XMIN, W.cstat[slot0 + c].xmin);
    }
    double Z = 0.0;
    for (int c = 0; c < nch; ++c) {
        ChunkStat cs = W.cstat[slot0 + c];
        if (cs.z != 0.0) Z += cs.z * exp((double)cs.m - (double)M);
    }

    RowInfo info;
    info.kind = KIND_UNFILTERED;
    info.nK = P.V;
    info.T = 0;
    info.ZK = Z;
    info.m = M;
    info.xmin = XMIN;
    info.idx0 = NONE;
    info.pad = 0;

    if (!filtered) {
        uint32_t idx;
        if (!md.sm) {
            uint64_t am = 0;
            for (int c = 0; c < nch; ++c)
                if (W.ccnt[slot0 + c] > 0) {
                    uint64_t v = W.cand[(int64_t)(slot0 + c) * SLOT];
                    am = v > am ? v : am;
                }
            idx = cidx(am);
        } else {
            float xr = -INFINITY;
            for (int c = 0; c < nch; ++c)
                if (W.cstat[slot0 + c].ridx != NONE) xr = fmaxf(xr, W.cstat[slot0 + c].rx);
            double br = -1.0;
            idx = NONE;
            for (int c = 0; c < nch; ++c) {
                ChunkStat cs = W.cstat[slot0 + c];
                if (cs.ridx == NONE) continue;
                double r = exp((double)cs.rx - (double)xr) / (double)cs.rqe;
                if (r > br || (r == br && cs.ridx < idx)) {
                    br = r;
                    idx = cs.ridx;
                }
            }
        }
        info.idx0 = idx;
        if (tid == 0) {
            P.out_idx[b] = (int64_t)idx;
            W.info[b] = info;
        }
        return;
    }

    // ---- candidates: exact top-kk over the row.  Sources 0..nch-1 are the
    // chunks' hand-overs, source NCH_MAX the row's redo slot, which replaces
    // the chunks in rmask.
    const uint32_t kk = md.tk ? (uint32_t)md.k : (uint32_t)min(P.guess, P.V);
    const uint32_t rmask = W.rmask[b];
    uint32_t scnt[NCH_MAX + 1];
    uint32_t N = 0;
#pragma unroll
    for (int c = 0; c <= NCH_MAX; ++c) {
        uint32_t n = 0;
        if (c == NCH_MAX) n = rmask ? (uint32_t)W.rcnt[b] : 0u;
        else if (c < nch && !((rmask >> c) & 1u)) n = (uint32_t)max(W.ccnt[slot0 + c], 0);
        scnt[c] = n;
        N += n;
    }
    constexpr int R2 = (NCH_MAX + 1) * SLOT / K2_THREADS;  // 18
    uint64_t v[R2];
    uint32_t vm = 0;
#pragma unroll
    for (int r = 0; r < R2; ++r) {
        constexpr int CPS = SLOT / K2_THREADS;  // rounds per source
        const int c = r / CPS;
        const uint32_t i = (uint32_t)((r % CPS) * K2_THREADS + tid);
        const bool ok = i < scnt[c];
        const uint64_t *src = (c == NCH_MAX) ? W.rcand + (int64_t)b * SLOT
                                             : W.cand + (int64_t)(slot0 + c) * SLOT;
        v[r] = ok ? src[i] : 0ull;
        if (ok) vm |= 1u << r;
    }
    const uint32_t nsel = min(kk, N);
    uint32_t km = vm;
    if (N > kk) {
        uint64_t prefix, pmask;
        wg_radix_select<K2_THREADS, R2>(v, vm, kk, S.hist, S.sel, S.sc64, prefix, pmask);
        km = 0;
#pragma unroll
        for (int r = 0; r < R2; ++r)
            if (((vm >> r) & 1u) && (v[r] & pmask) >= prefix) km |= 1u << r;
    }
    {
        uint32_t tot;
        uint32_t off = wg_excl_scan_u32<K2_THREADS>(__popc(km), S.sc, tot);
#pragma unroll
        for (int r = 0; r < R2; ++r)
            if ((km >> r) & 1u) S.srt[off++] = v[r];
    }
    const int npad = pow2_ceil((int)nsel);
    for (int i = nsel + tid; i < npad; i += K2_THREADS) S.srt[i] = 0ull;
    __syncthreads();
    bitonic_desc_reg<K2_THREADS>(S.srt, npad);

    // ---- softmax over the sorted candidates, in double
    const float x0 = cval(S.srt[0]);
    double e = 0.0;
    if ((uint32_t)tid < nsel) e = exp((double)cval(S.srt[tid]) - (double)x0);
    double tot_e;
    double incl = wg_excl_scan_f64<K2_THREADS>(e, S.scd, tot_e) + e;
    if ((uint32_t)tid < nsel) {
        S.ev[tid] = e;
        S.cs[tid] = incl;
    }
    __syncthreads();
    double Zc;
    if (md.tk) Zc = S.cs[nsel - 1];
    else Zc = (Z != 0.0) ? Z * exp((double)M - (double)x0) : tot_e;

    uint32_t nK = nsel;
    bool settled = true;
    if (md.tp) {
        const double pZ = (double)md.p * Zc;
        uint32_t first = NONE;
        if ((uint32_t)tid < nsel && S.cs[tid] >= pZ) first = (uint32_t)tid;
        first = wg_min_u32<K2_THREADS>(first, S.sc);
        if (md.tk) {
            nK = (first == NONE) ? nsel : first + 1;
        } else {
            // top-k guess (Ascend page, topP section): settled only when the
            // cutoff lies inside the guess with a safe margin on both sides.
            if (first == NONE) {
                settled = false;
            } else {
                double hi = S.cs[first] - pZ;
                double lo = (first == 0) ? INFINITY : pZ - S.cs[first - 1];
                settled = hi > GUESS_MARGIN * Zc && lo > GUESS_MARGIN * Zc;
                if (md.p <= 0.0f) settled = true;
                nK = first + 1;
            }
        }
    }
    info.m = x0;
    info.idx0 = cidx(S.srt[0]);
    if (!settled) {
        info.kind = KIND_FALLBACK;
        if (tid == 0) W.info[b] = info;
        return;
    }

    // ---- exponential race over K (or greedy)
    uint32_t idx = cidx(S.srt[0]);
    if (md.sm) {
        double r = -1.0;
        uint32_t id = NONE;
        if ((uint32_t)tid < nK) {
            id = cidx(S.srt[tid]);
            double den = (double)P.q[(int64_t)b * P.V + id] + (double)P.eps;
            double ei = S.ev[tid];
            r = (ei == 0.0) ? 0.0 : ei / den;
        }
        idx = wg_best_ratio<K2_THREADS>(r, id, S.scd, S.sci);
    }
    for (uint32_t i = tid; i < nK; i += K2_THREADS) W.klist[(int64_t)b * KMAX + i] = S.srt[i];
    info.kind = KIND_LIST;
    info.nK = (int32_t)nK;
    info.ZK = S.cs[nK - 1];
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
    uint32_t bm[K3_SEG / 32];
    // refinement levels: level 0 bins by value, later levels by key
    float lv_lo, lv_scale;
    uint32_t lv_bin[8];
    uint32_t lv_klo[8];
    uint64_t lv_span[8];
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
    float t = (x - lo) * scale;
    if (!(t >= 0.0f)) return 0u;
    if (t >= (float)(K3_BINS - 1)) return K3_BINS - 1;
    return (uint32_t)t;
}
__device__ __forceinline__ uint32_t bin_key(uint32_t key, uint32_t klo, uint64_t span) {
    uint64_t bi = ((uint64_t)(key - klo) * (uint64_t)K3_BINS) / span;
    return bi < (uint64_t)K3_BINS ? (uint32_t)bi : (uint32_t)(K3_BINS - 1);
}

// Boundary bucket of a mass histogram: walking the bins from the top, the
// bin where the running mass first reaches `need`.  Wave 0 sums 32 bins per
// lane; lane 0 then walks lane sums and that lane's bins with one running
// accumulator, so exactly one bin is chosen whatever the rounding.  Writes
// found[0] = bin, fd[0] = mass of the bins above it.  If rounding leaves
// `need` beyond the total, the lowest non-empty bin is chosen.
__device__ void find_bucket(const double *hm, const uint32_t *hc, double need, double *lane_sum,
                            uint32_t *found, double *fd) {
    constexpr int PER = K3_BINS / 64;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        double s = 0.0;
        for (int t = 0; t < PER; ++t) s += hm[K3_BINS - 1 - lane * PER - t];
        lane_sum[lane] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
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
        if (bin_key(k, S.lv_klo[l], S.lv_span[l]) != S.lv_bin[l]) return false;
    return true;
}

// Visit every element (x transformed, id j) of row b; f(x, j).
template <int DT, bool AL, bool XF, class F>
__device__ void row_pass(const KParams &P, int b, uint32_t *bm, F &&f) {
    const void *rowp = row_ptr(P, DT, b);
    const int64_t V = P.V;
    for (int64_t s0 = 0; s0 < V; s0 += K3_SEG) {
        const int64_t s1 = min(s0 + (int64_t)K3_SEG, V);
        if (P.pen) build_bitmap<K3_THREADS>(bm, s0, s1 - s0, P, b);
        for (int64_t j = s0 + (int64_t)threadIdx.x * VEC; j < s1; j += (int64_t)K3_THREADS * VEC) {
            int64_t rem = s1 - j;
            int nv = rem >= 8 ? 8 : (int)rem;
            float x[8];
            load8<DT, AL>(rowp, j, nv, x);
            uint32_t bits = 0;
            if (P.pen) {
                int64_t r = j - s0;
                bits = (bm[r >> 5] >> (r & 31)) & 0xffu;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (i < nv) f(xform<XF>(x[i], (bits >> i) & 1u, P), (uint32_t)(j + i));
        }
    }
    __syncthreads();
}

template <int DT, bool AL, bool XF>
__global__ __launch_bounds__(K3_THREADS) void k_fallback(KParams P, KPlan L, KWork W) {
    __shared__ FallbackShared S;
    const int tid = threadIdx.x;
    const int b = xcd_row(blockIdx.x, gridDim.x);
    RowInfo info = W.info[b];
    if (info.kind != KIND_FALLBACK) return;
    const Mode md = row_mode(P, b);
    const double m = (double)info.m;

    uint64_t Tstar;
    double ZK;
    if (md.p <= 0.0f) {
        Tstar = mkcomp(info.m, info.idx0);
        ZK = 1.0;
    } else {
        double above = 0.0, target = 0.0;
        int nlev = 0;
        int path = 0;  // 1 collect, 2 ties
        uint32_t bsel = 0, bcnt = 0, bklo = 0;
        for (int level = 0; level < 6; ++level) {
            // bin function of this level
            float lo = 0.0f, scale = 0.0f;
            uint32_t klo = 0;
            uint64_t span = 1;
            if (level == 0) {
                lo = info.xmin;
                scale = (info.m > info.xmin) ? (float)K3_BINS / (info.m - info.xmin) : 0.0f;
            } else {
                klo = S.lv_klo[level];
                span = S.lv_span[level];
            }
            for (int i = tid; i < K3_BINS; i += K3_THREADS) {
                S.hm[i] = 0.0;
                S.hc[i] = 0u;
                S.hlo[i] = NONE;
                S.hhi[i] = 0u;
            }
            __syncthreads();
            double zt = 0.0;
            row_pass<DT, AL, XF>(P, b, S.bm, [&](float x, uint32_t j) {
                if (!(x > -INFINITY)) return;
                uint32_t k = f2key(x);
                if (!in_play(S, x, k, nlev)) return;
                double e = exp((double)x - m);
                if (level == 0) zt += e;
                uint32_t bi = (level == 0) ? bin_value(x, lo, scale) : bin_key(k, klo, span);
                atomicAdd(&S.hm[bi], e);
                atomicAdd(&S.hc[bi], 1u);
                atomicMin(&S.hlo[bi], k);
                atomicMax(&S.hhi[bi], k);
            });
            if (level == 0) {
                double Z = wg_sum_f64<K3_THREADS>(zt, S.scd);
                target = (double)md.p * Z;
            }
            find_bucket(S.hm, S.hc, target - above, S.lane_sum, S.found, S.fd);
            const uint32_t fb = S.found[0];
            const double bbefore = S.fd[0];
            __syncthreads();
            above += bbefore;
            bsel = fb;
            bcnt = S.hc[fb];
            bklo = S.hlo[fb];
            const uint32_t bkhi = S.hhi[fb];
            __syncthreads();
            if (tid == 0) {
                if (level == 0) {
                    S.lv_lo = lo;
                    S.lv_scale = scale;
                }
                S.lv_bin[level] = fb;
                if (level + 1 < 8) {
                    S.lv_klo[level + 1] = bklo;
                    S.lv_span[level + 1] = (uint64_t)(bkhi - bklo) + 1ull;
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
        if (path == 1) {
            if (tid == 0) S.counter = 0;
            __syncthreads();
            row_pass<DT, AL, XF>(P, b, S.bm, [&](float x, uint32_t j) {
                if (!(x > -INFINITY)) return;
                uint32_t k = f2key(x);
                if (!in_play(S, x, k, nlev)) return;
                uint32_t pos = atomicAdd(&S.counter, 1u);
                if (pos < (uint32_t)K3_COLLECT) S.coll[pos] = mkcomp(x, j);
            });
            const int n = (int)min(S.counter, (uint32_t)K3_COLLECT);
            const int npad = pow2_ceil(n < 1 ? 1 : n);
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
                ei[t] = (i < n) ? exp((double)cval(S.coll[i]) - m) : 0.0;
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
            uint32_t fi = wg_min_u32<K3_THREADS>(first, S.sc);
            if (fi == NONE) fi = (uint32_t)(n > 0 ? n - 1 : 0);  // rounding: whole bucket
            Tstar = (n > 0) ? S.coll[fi] : mkcomp(info.m, info.idx0);
            // ZK: mass of every kept element = above + bucket prefix through fi
            double s = 0.0;
#pragma unroll
            for (int t = 0; t < PER; ++t) {
                int i = tid * PER + t;
                if (i <= (int)fi && i < n) s += ei[t];
            }
            ZK = above + wg_sum_f64<K3_THREADS>(s, S.scd);
        } else {
            // every bucket member has the same value: take the c members with
            // the smallest vocab ids
            const float xt = key2f(bklo);
            const double et = exp((double)xt - m);
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
            Tstar = mkcomp(xt, S.found[1]);
            ZK = above + (double)cneed * et;
        }
    }

    // ---- exponential race over K = { comp >= T* }, or greedy
    uint32_t idx = info.idx0;
    if (md.sm) {
        Race rc;
        rc.x = -INFINITY; rc.qe = 1.0f; rc.idx = NONE;
        const float *rowq = P.q + (int64_t)b * P.V;
        row_pass<DT, AL, XF>(P, b, S.bm, [&](float x, uint32_t j) {
            if (mkcomp(x, j) >= Tstar) race_offer(rc, x, rowq[j] + P.eps, j);
        });
        Race r = wg_race<K3_THREADS>(rc, S.scx, S.scq, S.sci);
        idx = r.idx;
    }
    if (tid == 0) {
        P.out_idx[b] = (int64_t)idx;
        info.kind = KIND_THRESH;
        info.T = Tstar;
        info.ZK = ZK;
        W.info[b] = info;
    }
}

// ================================================================== k_dense

// Dense filtered logits (and optional probabilities) of one 32768-element
// tile of one row.  Rows with a kept list: the tile is written from a bitmap
// of the kept positions and the kept values placed by their rank among the
// set bits (no read of the logits, full-line stores).  Rows whose kept set is
// a threshold (after the full-row search) re-read and re-transform the tile.

struct DenseShared {
    uint32_t tb[TILE4 / 32];    // kept positions in the tile
    uint32_t wpre[TILE4 / 32];  // set bits before each word
    float lval[KMAX];           // kept values by rank
    uint32_t sc[16];
};

template <int DT, bool AL, bool XF>
__global__ __launch_bounds__(K4_THREADS) void k_dense(KParams P, KPlan L, KWork W) {
    __shared__ DenseShared S;
    extern __shared__ uint32_t bm[];  // penalty bitmap of the tile
    const int tid = threadIdx.x;
    const int b = blockIdx.x / L.nt4, t = blockIdx.x % L.nt4;
    const int64_t V = P.V;
    const int64_t t0 = (int64_t)t * TILE4, t1 = min(t0 + (int64_t)TILE4, V);
    const RowInfo info = W.info[b];
    const bool want_l = (P.flags & NEED_LOGITS) && P.out_logits;
    const bool want_p = (P.flags & NEED_PROBS) && P.out_probs;
    if (info.kind == KIND_UNFILTERED && !want_p) return;
    float *ol = want_l ? P.out_logits + (int64_t)b * V : nullptr;
    float *op = want_p ? P.out_probs + (int64_t)b * V : nullptr;
    const double m = (double)info.m, ZK = info.ZK;
    constexpr int G = TILE4 / (K4_THREADS * VEC);  // groups of 8 per thread
    constexpr int WPT = TILE4 / 32 / K4_THREADS;   // bitmap words per thread

    if (info.kind == KIND_LIST) {
#pragma unroll
        for (int w = 0; w < WPT; ++w) S.tb[tid * WPT + w] = 0u;
        __syncthreads();
        const uint64_t *kl = W.klist + (int64_t)b * KMAX;
        const int nK = info.nK;
        for (int i = tid; i < nK; i += K4_THREADS) {
            const int64_t j = cidx(kl[i]);
            if (j >= t0 && j < t1) {
                const int r = (int)(j - t0);
                atomicOr(&S.tb[r >> 5], 1u << (r & 31));
            }
        }
        __syncthreads();
        uint32_t cnt = 0;
#pragma unroll
        for (int w = 0; w < WPT; ++w) cnt += __popc(S.tb[tid * WPT + w]);
        uint32_t tot;
        uint32_t run = wg_excl_scan_u32<K4_THREADS>(cnt, S.sc, tot);
#pragma unroll
        for (int w = 0; w < WPT; ++w) {
            S.wpre[tid * WPT + w] = run;
            run += __popc(S.tb[tid * WPT + w]);
        }
        __syncthreads();
        for (int i = tid; i < nK; i += K4_THREADS) {
            const uint64_t cv = kl[i];
            const int64_t j = cidx(cv);
            if (j >= t0 && j < t1) {
                const int r = (int)(j - t0);
                const uint32_t below = S.tb[r >> 5] & ((1u << (r & 31)) - 1u);
                S.lval[S.wpre[r >> 5] + __popc(below)] = cval(cv);
            }
        }
        __syncthreads();
#pragma unroll 4
        for (int g = 0; g < G; ++g) {
            const int r0 = (g * K4_THREADS + tid) * VEC;
            const int64_t j = t0 + r0;
            const int nv = group_nv(j, t1);
            if (nv == 0) continue;
            const uint32_t word = S.tb[r0 >> 5];
            const uint32_t bits = (word >> (r0 & 31)) & 0xffu;
            float xv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) xv[i] = -INFINITY;
            if (bits) {
                const uint32_t base = S.wpre[r0 >> 5] + __popc(word & ((1u << (r0 & 31)) - 1u));
                uint32_t k = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if ((bits >> i) & 1u) xv[i] = S.lval[base + k++];
            }
            if (want_l) store8<AL>(ol, j, nv, xv);
            if (want_p) {
                float o[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    o[i] = ((bits >> i) & 1u) ? (float)(exp((double)xv[i] - m) / ZK) : 0.0f;
                store8<AL>(op, j, nv, o);
            }
        }
        return;
    }
    if (info.kind != KIND_THRESH && info.kind != KIND_UNFILTERED) return;
    // K = { comp >= T } (T = 0 keeps the whole row): re-read the tile
    if (XF && P.pen) build_bitmap<K4_THREADS>(bm, t0, t1 - t0, P, b);
    const void *rowp = row_ptr(P, DT, b);
    const uint64_t T = info.T;
    for (int g = 0; g < G; ++g) {
        const int r0 = (g * K4_THREADS + tid) * VEC;
        const int64_t j = t0 + r0;
        const int nv = group_nv(j, t1);
        if (nv == 0) continue;
        float x[8];
        load8<DT, AL>(rowp, j, nv, x);
        const uint32_t bits = pen_bits<XF>(bm, r0, P);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = xform<XF>(x[i], (bits >> i) & 1u, P);
        if (want_l && info.kind == KIND_THRESH) {
            float o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                o[i] = (mkcomp(x[i], (uint32_t)(j + i)) >= T) ? x[i] : -INFINITY;
            store8<AL>(ol, j, nv, o);
        }
        if (want_p) {
            float o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                o[i] = (mkcomp(x[i], (uint32_t)(j + i)) >= T)
                           ? (float)(exp((double)x[i] - m) / ZK)
                           : 0.0f;
            store8<AL>(op, j, nv, o);
        }
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

hipError_t launch_stream(const KParams &p, const KPlan &l, const KWork &w, int dtype, bool al,
                         hipStream_t s) {
    const bool xf = any_transform(p);
    dim3 grid((unsigned)((int64_t)p.B * l.nch)), block(K1_THREADS);
    size_t sh = p.pen ? (size_t)((l.chunk_len + 31) / 32) * 4 : 0;
    return SMP_PICK(k_stream, grid, block, sh);
}

hipError_t launch_select(const KParams &p, const KPlan &l, const KWork &w, int dtype, bool al,
                         hipStream_t s) {
    const bool xf = any_transform(p);
    dim3 grid((unsigned)((int64_t)p.B * l.nch)), block(SEL_THREADS);
    size_t sh = p.pen ? (size_t)((l.chunk_len + 31) / 32) * 4 : 0;
    return SMP_PICK(k_select, grid, block, sh);
}

hipError_t launch_fix(const KParams &p, const KPlan &l, const KWork &w, int dtype, bool al,
                      hipStream_t s) {
    const bool xf = any_transform(p);
    dim3 grid((unsigned)p.B), block(SEL_THREADS);
    size_t sh = p.pen ? (size_t)((l.chunk_len + 31) / 32) * 4 : 0;
    return SMP_PICK(k_fix, grid, block, sh);
}

hipError_t launch_rows(const KParams &p, const KPlan &l, const KWork &w, hipStream_t s) {
    return launch(k_rows, dim3((unsigned)p.B), dim3(K2_THREADS), 0, s, p, l, w);
}

hipError_t launch_fallback(const KParams &p, const KPlan &l, const KWork &w, int dtype, bool al,
                           hipStream_t s) {
    const bool xf = any_transform(p);
    dim3 grid((unsigned)p.B), block(K3_THREADS);
    return SMP_PICK(k_fallback, grid, block, 0);
}

hipError_t launch_dense(const KParams &p, const KPlan &l, const KWork &w, int dtype, bool al,
                        hipStream_t s) {
    const bool xf = any_transform(p);
    dim3 grid((unsigned)((int64_t)p.B * l.nt4)), block(K4_THREADS);
    size_t sh = p.pen ? (size_t)(TILE4 / 32) * 4 : 0;
    return SMP_PICK(k_dense, grid, block, sh);
}

#undef SMP_PICK

}  // namespace smp
