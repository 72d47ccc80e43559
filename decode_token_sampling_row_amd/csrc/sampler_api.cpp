#include <algorithm>
// C ABI of the batched logits sampler: argument checks, workspace, planning
// and kernel launches.  The operation itself is defined in sampler.h.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <new>

#include "sampler.h"
#include "sampler_internal.h"

using namespace smp;

constexpr int PROF_KERNELS = SAMPLER_PROFILE_SLOTS;
constexpr int PROF_RING = 64;

// The settings a call runs with: the handle's, or those given to
// sampler_run_static.
struct Config {
    int32_t max_batch;
    int32_t rows_per_launch;  // 0 = automatic
    int32_t vocab;
    int32_t dtype;
    int32_t guess;
    int32_t seg;
    bool seg_auto;  // the tile length is chosen per call (auto_seg)
    int32_t cus;    // compute units of the device
};

struct sampler_s {
    Config cfg;
    int device;
    KWork ws;
    void *ws_base;
    // profiling: a ring of PROF_RING calls, PROF_KERNELS + 1 events each
    hipEvent_t ev[PROF_RING][PROF_KERNELS + 1];
    bool events_made;
    bool events_ok;
    int nprof;   // profiled calls since the last read
    bool launched[PROF_RING][PROF_KERNELS];
};

namespace {

constexpr int32_t DEFAULT_GUESS = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Options and sizes common to sampler_create and sampler_run_static.
int make_config(Config &c, int32_t max_batch, int32_t vocab, int32_t dtype,
                const sampler_opts *opts) {
    if (max_batch < 1 || vocab < 1 || vocab > SAMPLER_VOCAB_MAX) return SAMPLER_EINVAL;
    if (dtype != SAMPLER_F32 && dtype != SAMPLER_BF16) return SAMPLER_EINVAL;
    c.max_batch = max_batch;
    c.vocab = vocab;
    c.dtype = dtype;
    c.guess = DEFAULT_GUESS;
    c.seg = SEG_DEFAULT;
    c.seg_auto = true;
    c.rows_per_launch = 0;
    c.cus = 1;
    if (opts) {
        if (opts->topk_guess < 0 || opts->topk_guess > SAMPLER_TOPK_MAX) return SAMPLER_EINVAL;
        if (opts->segment_len != 0 &&
            (opts->segment_len < SEG_MIN || opts->segment_len > SEG_MAX ||
             opts->segment_len % SEG_MIN != 0))
            return SAMPLER_EINVAL;
        if (opts->rows_per_launch < 0) return SAMPLER_EINVAL;
        if (opts->topk_guess) c.guess = opts->topk_guess;
        if (opts->segment_len) {
            c.seg = opts->segment_len;
            c.seg_auto = false;
        }
        c.rows_per_launch = opts->rows_per_launch;
    }
    return SAMPLER_OK;
}

// The tile length of a call of batch rows.
int32_t call_seg(const Config &c, int32_t batch) {
    return c.seg_auto ? auto_seg(batch, c.vocab, c.cus) : c.seg;
}

// The workspace of B rows and `tiles` (row, tile) records laid out from base
// (null: only sized).  Returns its size in bytes.
size_t layout_workspace(size_t B, size_t tiles, const KPlan &plan, char *base, KWork *w) {
    size_t off = 0;
    const size_t o_cand = off;
    off = align_up(off + B * ROWCAP * sizeof(uint64_t), 256);
    const size_t o_wcnt = off;
    off = align_up(off + tiles * 4 * sizeof(uint32_t), 256);  // one per wave sub-slot
    const size_t o_cstat = off;
    off = align_up(off + tiles * 4 * sizeof(ChunkStat), 256);
    const size_t o_info = off;
    off = align_up(off + B * sizeof(RowInfo), 256);
    const size_t o_klist = off;
    off = align_up(off + B * KMAX * sizeof(uint64_t), 256);
    const size_t o_ktoff = off;
    off = align_up(off + B * ((size_t)plan.ntd + 1) * sizeof(uint32_t), 256);
    const size_t o_rowthr = off;
    off = align_up(off + B * sizeof(float), 256);
    const size_t o_rowref = off;
    off = align_up(off + B * sizeof(float), 256);
    const size_t o_rowlo = off;
    off = align_up(off + B * sizeof(float), 256);
    const size_t o_fbcnt = off;
    off = align_up(off + sizeof(uint32_t), 256);
    const size_t o_fblist = off;
    off = align_up(off + B * sizeof(uint32_t), 256);
    const size_t o_fbsync = off;
    off = align_up(off + (size_t)FB_GRID * FB_SYNC_WORDS * sizeof(uint32_t), 256);
    const size_t o_fbpart = off;
    off = align_up(off + (size_t)fb_grid((int)B) * FB_PART_BYTES, 256);
    if (base) {
        w->cand = (uint64_t *)(base + o_cand);
        w->wcnt = (uint32_t *)(base + o_wcnt);
        w->cstat = (ChunkStat *)(base + o_cstat);
        w->info = (RowInfo *)(base + o_info);
        w->klist = (uint64_t *)(base + o_klist);
        w->ktoff = (uint32_t *)(base + o_ktoff);
        w->rowthr = (float *)(base + o_rowthr);
        w->rowref = (float *)(base + o_rowref);
        w->rowlo = (float *)(base + o_rowlo);
        w->fbcnt = (uint32_t *)(base + o_fbcnt);
        w->fblist = (uint32_t *)(base + o_fblist);
        w->fbsync = (uint32_t *)(base + o_fbsync);
        w->fbpart = base + o_fbpart;
    }
    return off;
}

int check_args(const Config &c, int32_t batch, const sampler_args *a) {
    if (a == nullptr) return SAMPLER_EINVAL;
    if (batch < 0 || batch > c.max_batch) return SAMPLER_EINVAL;
    if (batch == 0) return SAMPLER_OK;
    if (a->logits == nullptr || a->out_idx == nullptr) return SAMPLER_EINVAL;
    if (a->ld < c.vocab) return SAMPLER_EINVAL;
    if (!(a->temperature > 0.0f) || !isfinite(a->temperature)) return SAMPLER_EINVAL;
    if (!(a->repetition_penalty > 0.0f) || !isfinite(a->repetition_penalty))
        return SAMPLER_EINVAL;
    if (!(a->eps >= 0.0f) || !isfinite(a->eps)) return SAMPLER_EINVAL;
    const uint32_t known = SAMPLER_NEED_LOGITS | SAMPLER_NEED_PROBS | SAMPLER_TOPK_TIES |
                           SAMPLER_APPEND_HISTORY | SAMPLER_PROFILE;
    if (a->flags & ~known) return SAMPLER_EINVAL;
    if ((a->flags & SAMPLER_NEED_LOGITS) && a->out_logits == nullptr) return SAMPLER_EINVAL;
    if ((a->flags & SAMPLER_NEED_PROBS) && a->out_probs == nullptr) return SAMPLER_EINVAL;
    if ((a->penalty_ids == nullptr) != (a->penalty_offsets == nullptr)) return SAMPLER_EINVAL;
    if (a->penalty_len != nullptr && a->penalty_ids == nullptr) return SAMPLER_EINVAL;
    if ((a->flags & SAMPLER_APPEND_HISTORY) && a->penalty_len == nullptr) return SAMPLER_EINVAL;
    if (a->finished != nullptr && (a->eos_id < 0 || a->eos_id >= c.vocab)) return SAMPLER_EINVAL;
    if (a->row_flags == nullptr && a->q == nullptr && a->u == nullptr) return SAMPLER_EINVAL;
    return SAMPLER_OK;
}

// Per-kernel HIP events of a profiled call (none for sampler_run_static).
struct Marks {
    hipEvent_t *ev;  // PROF_KERNELS + 1 events, or null
    bool *launched;  // PROF_KERNELS flags, or null
    void mark(int i, hipStream_t st) const {
        if (ev) (void)hipEventRecord(ev[i], st);
    }
    void done(int i) const {
        if (launched) launched[i] = true;
    }
};

// The launch sequence of one call over batch rows with workspace ws.
int run_call(const Config &c, const KWork &ws, int32_t batch, const sampler_args *a,
             hipStream_t st, const Marks &mk) {
    KParams p;
    memset(&p, 0, sizeof p);
    p.logits = a->logits;
    p.ld = a->ld;
    p.top_k = a->top_k;
    p.top_p = a->top_p;
    p.q = a->q;
    p.u = a->u;
    p.ids = a->penalty_ids;
    p.offsets = a->penalty_offsets;
    p.plen = a->penalty_len;
    p.row_flags = a->row_flags;
    p.out_idx = a->out_idx;
    p.out_logits = (a->flags & SAMPLER_NEED_LOGITS) ? a->out_logits : nullptr;
    p.out_probs = (a->flags & SAMPLER_NEED_PROBS) ? a->out_probs : nullptr;
    p.eps = a->eps;
    p.temperature = a->temperature;
    p.rho = a->repetition_penalty;
    p.flags = a->flags & (SAMPLER_NEED_LOGITS | SAMPLER_NEED_PROBS | SAMPLER_TOPK_TIES);
    p.B = batch;
    p.V = c.vocab;
    p.guess = c.guess;
    p.pen = (a->repetition_penalty != 1.0f && a->penalty_ids != nullptr) ? 1 : 0;

    const KPlan l = make_plan(c.vocab, call_seg(c, batch), c.cus);
    const int esize = c.dtype == SAMPLER_BF16 ? 2 : 4;
    const bool al = aligned16(a->logits) && ((a->ld * esize) % 16) == 0 &&
                    (c.vocab % 4) == 0 && (a->q == nullptr || aligned16(a->q)) &&
                    (p.out_logits == nullptr || aligned16(p.out_logits)) &&
                    (p.out_probs == nullptr || aligned16(p.out_probs));
    const bool filtering = a->top_k != nullptr || a->top_p != nullptr;

    // Rows go in chunks small enough for every grid (at most 2^23 workgroups
    // of at most 1024 threads); each kernel runs over all chunks before the
    // next kernel starts, so the per-kernel profile spans stay contiguous.
    const int64_t max_wg = (int64_t)1 << 23;
    int64_t lim = std::max<int64_t>(1, max_wg / std::max(l.nt, l.ntd));
    if (c.rows_per_launch > 0) lim = std::min<int64_t>(lim, c.rows_per_launch);
    const int chunk = (int)std::min<int64_t>(batch, lim);
    auto each = [&](auto &&launcher) -> bool {
        for (int c0 = 0; c0 < batch; c0 += chunk) {
            KParams pc = p;
            pc.b0 = c0;
            pc.B = std::min(chunk, batch - c0);
            if (launcher(pc) != hipSuccess) return false;
        }
        return true;
    };

    mk.mark(0, st);
    if (filtering) {
        if (!each([&](const KParams &pc) { return launch_plan(pc, l, ws, c.dtype, al, st); }))
            return SAMPLER_EHIP;
        mk.done(0);
    }
    mk.mark(1, st);
    if (!each([&](const KParams &pc) { return launch_pass(pc, l, ws, c.dtype, al, st); }))
        return SAMPLER_EHIP;
    mk.done(1);
    mk.mark(2, st);
    if (!each([&](const KParams &pc) { return launch_rows(pc, l, ws, st); })) return SAMPLER_EHIP;
    mk.done(2);
    mk.mark(3, st);
    if (filtering || a->u != nullptr) {
        // one launch over the queue the merge filled, whatever the chunks
        if (launch_fallback(p, l, ws, c.dtype, al, st) != hipSuccess) return SAMPLER_EHIP;
        mk.done(3);
    }
    mk.mark(4, st);
    if (p.out_probs || (p.out_logits && filtering)) {
        if (!each([&](const KParams &pc) { return launch_dense(pc, l, ws, c.dtype, al, st); }))
            return SAMPLER_EHIP;
        mk.done(4);
    }
    mk.mark(5, st);
    const bool append = (a->flags & SAMPLER_APPEND_HISTORY) != 0;
    if (a->finished || append || a->counts) {
        // after every kernel that reads the history or writes out_idx
        EpiParams e;
        e.out_idx = a->out_idx;
        e.finished = a->finished;
        e.eos = a->eos_id;
        e.ids = a->penalty_ids;
        e.offsets = a->penalty_offsets;
        e.len = a->penalty_len;
        e.counts = a->counts;
        e.B = batch;
        e.append = append ? 1 : 0;
        if (launch_epilogue(e, st) != hipSuccess) return SAMPLER_EHIP;
        mk.done(5);
    }
    mk.mark(6, st);
    return SAMPLER_OK;
}

}  // namespace

extern "C" {

const char *sampler_strerror(int code) {
    switch (code) {
        case SAMPLER_OK: return "ok";
        case SAMPLER_EINVAL: return "invalid argument";
        case SAMPLER_ENOMEM: return "device workspace allocation failed";
        case SAMPLER_EHIP: return "HIP runtime error";
        default: return "unknown error";
    }
}

int sampler_create(sampler_t **h, int32_t max_batch, int32_t vocab, int32_t dtype,
                   const sampler_opts *opts) {
    if (h == nullptr) return SAMPLER_EINVAL;
    *h = nullptr;
    Config cfg;
    const int rc = make_config(cfg, max_batch, vocab, dtype, opts);
    if (rc != SAMPLER_OK) return rc;

    sampler_s *s = new (std::nothrow) sampler_s();
    if (!s) return SAMPLER_ENOMEM;
    if (hipGetDevice(&s->device) != hipSuccess ||
        hipDeviceGetAttribute(&cfg.cus, hipDeviceAttributeMultiprocessorCount, s->device) !=
            hipSuccess) {
        delete s;
        return SAMPLER_EHIP;
    }
    if (cfg.cus < 1) cfg.cus = 1;
    s->cfg = cfg;
    // tile records for every batch up to max_batch, at the fixed tile length
    // or at any the call may choose (auto_seg)
    const KPlan plan = make_plan(vocab, cfg.seg, cfg.cus);
    size_t tiles = (size_t)max_batch * (size_t)plan.nt;
    if (cfg.seg_auto) tiles = std::max(tiles, (size_t)AUTO_WG_PER_CU * (size_t)cfg.cus);
    const size_t bytes = layout_workspace((size_t)max_batch, tiles, plan, nullptr, nullptr);
    void *base = nullptr;
    hipError_t e = hipMalloc(&base, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        delete s;
        return e == hipErrorOutOfMemory ? SAMPLER_ENOMEM : SAMPLER_EHIP;
    }
    s->ws_base = base;
    (void)layout_workspace((size_t)max_batch, tiles, plan, (char *)base, &s->ws);
    s->events_made = false;
    s->events_ok = false;
    s->nprof = 0;
    *h = s;
    return SAMPLER_OK;
}

int sampler_check(const sampler_t *h, int32_t batch, const sampler_args *a) {
    if (h == nullptr) return SAMPLER_EINVAL;
    return check_args(h->cfg, batch, a);
}

int sampler_run(sampler_t *h, int32_t batch, const sampler_args *a, void *stream) {
    int rc = sampler_check(h, batch, a);
    if (rc != SAMPLER_OK) return rc;
    if (batch == 0) return SAMPLER_OK;
    hipStream_t st = (hipStream_t)stream;

    bool prof = (a->flags & SAMPLER_PROFILE) != 0;
    if (prof && !h->events_made) {
        h->events_made = true;
        h->events_ok = true;
        for (int r = 0; r < PROF_RING; ++r)
            for (int i = 0; i <= PROF_KERNELS; ++i)
                if (hipEventCreate(&h->ev[r][i]) != hipSuccess) h->events_ok = false;
    }
    prof = prof && h->events_ok;
    const int slot = h->nprof % PROF_RING;
    bool *launched = h->launched[slot];
    for (int i = 0; i < PROF_KERNELS; ++i) launched[i] = false;
    Marks mk;
    mk.ev = prof ? h->ev[slot] : nullptr;
    mk.launched = launched;
    rc = run_call(h->cfg, h->ws, batch, a, st, mk);
    if (rc != SAMPLER_OK) return rc;
    if (prof) ++h->nprof;
    return SAMPLER_OK;
}

int sampler_run_static(int32_t batch, int32_t vocab, int32_t dtype, const sampler_opts *opts,
                       const sampler_args *a, void *stream) {
    Config cfg;
    int rc = make_config(cfg, batch < 1 ? 1 : batch, vocab, dtype, opts);
    if (rc != SAMPLER_OK) return rc;
    if (batch < 0) return SAMPLER_EINVAL;
    rc = check_args(cfg, batch, a);
    if (rc != SAMPLER_OK) return rc;
    if (a->flags & SAMPLER_PROFILE) return SAMPLER_EINVAL;  // no events: nothing is created
    if (batch == 0) return SAMPLER_OK;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess ||
        hipDeviceGetAttribute(&cfg.cus, hipDeviceAttributeMultiprocessorCount, device) !=
            hipSuccess)
        return SAMPLER_EHIP;
    if (cfg.cus < 1) cfg.cus = 1;
    const KPlan plan = make_plan(vocab, call_seg(cfg, batch), cfg.cus);
    const size_t tiles = (size_t)batch * (size_t)plan.nt;
    const size_t bytes = layout_workspace((size_t)batch, tiles, plan, nullptr, nullptr);
    if (bytes > (size_t)SAMPLER_STATIC_SCRATCH_BYTES) return SAMPLER_EINVAL;
    void *base = nullptr;
    if (static_scratch(device, &base) != hipSuccess) return SAMPLER_EHIP;
    KWork ws;
    (void)layout_workspace((size_t)batch, tiles, plan, (char *)base, &ws);
    Marks mk;
    mk.ev = nullptr;
    mk.launched = nullptr;
    return run_call(cfg, ws, batch, a, (hipStream_t)stream, mk);
}

int sampler_profile(sampler_t *h, float *ms, int32_t n) {
    if (h == nullptr || ms == nullptr || n < 0) return SAMPLER_EINVAL;
    if (h->nprof == 0) return SAMPLER_EINVAL;
    const int calls = h->nprof < PROF_RING ? h->nprof : PROF_RING;
    const int last = (h->nprof - 1) % PROF_RING;
    if (hipEventSynchronize(h->ev[last][PROF_KERNELS]) != hipSuccess) return SAMPLER_EHIP;
    const int w = n < PROF_KERNELS ? n : PROF_KERNELS;
    for (int i = 0; i < w; ++i) {
        double sum = 0.0;
        for (int r = 0; r < calls; ++r) {
            float t = 0.0f;
            if (h->launched[r][i] &&
                hipEventElapsedTime(&t, h->ev[r][i], h->ev[r][i + 1]) != hipSuccess)
                return SAMPLER_EHIP;
            sum += h->launched[r][i] ? t : 0.0f;
        }
        ms[i] = (float)(sum / calls);
    }
    h->nprof = 0;
    return w;
}

int sampler_destroy(sampler_t *h) {
    if (h == nullptr) return SAMPLER_OK;
    int rc = SAMPLER_OK;
    if (h->ws_base && hipFree(h->ws_base) != hipSuccess) rc = SAMPLER_EHIP;
    if (h->events_made)
        for (int r = 0; r < PROF_RING; ++r)
            for (int i = 0; i <= PROF_KERNELS; ++i)
                if (h->ev[r][i]) (void)hipEventDestroy(h->ev[r][i]);
    delete h;
    return rc;
}

}  // extern "C"
