// CPU check of the C ABI's host code (sampler_api.cpp): argument checks,
// create / destroy error paths, workspace layout, row chunking and the launch
// sequence, built with AddressSanitizer and UBSan by the test suite.
//
// The HIP runtime calls the host code makes and the kernel launchers are
// replaced here by recording stand-ins: device allocations are host heap
// blocks of exactly the requested size, and each launcher writes every
// workspace entry the launched rows may use (so a layout that gives a row
// less room than its kernels index is an AddressSanitizer error) and checks
// the launch shape (rows within the call, grids within the chunk limit).
// Any failed check prints its case and exits non-zero.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <sanitizer/asan_interface.h>

#include <algorithm>
#include <vector>

#include "sampler.h"
#include "sampler_internal.h"

using namespace smp;

static int failures = 0;
#define CHECK(cond, ...)                                                            \
    do {                                                                            \
        if (!(cond)) {                                                              \
            if (failures < 30) {                                                    \
                fprintf(stderr, "FAIL %s:%d: %s | ", __FILE__, __LINE__, #cond);    \
                fprintf(stderr, __VA_ARGS__);                                       \
                fprintf(stderr, "\n");                                              \
            }                                                                       \
            ++failures;                                                             \
        }                                                                           \
    } while (0)

// ---------------------------------------------------------------------------
// Recording stand-in for the HIP runtime.

struct Block {
    char *p;
    size_t n;
};
static std::vector<Block> live;      // allocations not yet freed
static int n_events_live = 0;
static int fail_get_device = 0;      // next hipGetDevice fails
static int fail_attribute = 0;       // next hipDeviceGetAttribute fails
static hipError_t fail_malloc = hipSuccess;
static int fail_event_create = 0;    // hipEventCreate fails after this many more (0: never)
static int fail_launch_kernel = -1;  // kernel slot whose launch fails (-1: none)
static int cus = 256;

struct FakeEvent {
    int recorded;
};

extern "C" {
hipError_t hipGetDevice(int *d) {
    if (fail_get_device) {
        fail_get_device = 0;
        return hipErrorNoDevice;
    }
    *d = 0;
    return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t a, int dev) {
    CHECK(dev == 0, "device %d", dev);
    if (fail_attribute) {
        fail_attribute = 0;
        return hipErrorInvalidValue;
    }
    CHECK(a == hipDeviceAttributeMultiprocessorCount, "attribute %d", (int)a);
    *v = cus;
    return hipSuccess;
}
hipError_t hipMalloc(void **p, size_t n) {
    if (fail_malloc != hipSuccess) {
        const hipError_t e = fail_malloc;
        fail_malloc = hipSuccess;
        *p = nullptr;
        return e;
    }
    const size_t r = (n + 255) / 256 * 256;
    char *b = (char *)aligned_alloc(256, r == 0 ? 256 : r);
    if (!b) return hipErrorOutOfMemory;
    // poison the tail that rounding added, so only the n bytes asked for are usable
    ASAN_POISON_MEMORY_REGION(b + n, r - n);
    live.push_back({b, n});
    *p = b;
    return hipSuccess;
}
hipError_t hipFree(void *p) {
    for (size_t i = 0; i < live.size(); ++i)
        if (live[i].p == p) {
            ASAN_UNPOISON_MEMORY_REGION(live[i].p, (live[i].n + 255) / 256 * 256);
            free(p);
            live.erase(live.begin() + (long)i);
            return hipSuccess;
        }
    CHECK(p == nullptr, "hipFree of an unknown pointer");
    return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipEventCreate(hipEvent_t *e) {
    if (fail_event_create && --fail_event_create == 0) return hipErrorOutOfMemory;
    *e = reinterpret_cast<hipEvent_t>(new FakeEvent{0});
    ++n_events_live;
    return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t e) {
    delete reinterpret_cast<FakeEvent *>(e);
    --n_events_live;
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t) {
    reinterpret_cast<FakeEvent *>(e)->recorded++;
    return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t e) {
    CHECK(reinterpret_cast<FakeEvent *>(e)->recorded > 0, "synchronize on an unrecorded event");
    return hipSuccess;
}
hipError_t hipEventElapsedTime(float *ms, hipEvent_t a, hipEvent_t b) {
    CHECK(reinterpret_cast<FakeEvent *>(a)->recorded > 0 &&
              reinterpret_cast<FakeEvent *>(b)->recorded > 0,
          "elapsed time between unrecorded events");
    *ms = 0.25f;
    return hipSuccess;
}
}  // extern "C"

// ---------------------------------------------------------------------------
// Recording launchers.

struct Launch {
    int kernel;  // profile slot: 0 plan, 1 pass, 2 rows, 3 fallback, 4 dense, 5 epilogue
    int b0, B;
    int dtype;
    bool aligned;
    KPlan plan;
};
static std::vector<Launch> launches;
static int call_batch = 0;  // rows of the call being checked
static std::vector<unsigned char> static_area;

static bool inside(const void *p, size_t n, const char **what) {
    const char *c = (const char *)p;
    for (const Block &b : live)
        if (c >= b.p && c + n <= b.p + b.n) return true;
    if (!static_area.empty() && c >= (const char *)static_area.data() &&
        c + n <= (const char *)static_area.data() + static_area.size())
        return true;
    (void)what;
    return false;
}

// Write every workspace entry rows [0, rows) may use, after checking it lies
// inside one allocation; the regions must not overlap.
static void touch_workspace(const KPlan &l, const KWork &w, int rows, int kernel) {
    struct R {
        const char *name;
        void *p;
        size_t n;
    } r[] = {
        {"cand", w.cand, (size_t)rows * ROWCAP * sizeof(uint64_t)},
        {"wcnt", w.wcnt, (size_t)rows * l.nt * 4 * sizeof(uint32_t)},
        {"cstat", w.cstat, (size_t)rows * l.nt * 4 * sizeof(ChunkStat)},
        {"info", w.info, (size_t)rows * sizeof(RowInfo)},
        {"klist", w.klist, (size_t)rows * KMAX * sizeof(uint64_t)},
        {"ktoff", w.ktoff, (size_t)rows * (l.ntd + 1) * sizeof(uint32_t)},
        {"rowthr", w.rowthr, (size_t)rows * sizeof(float)},
        {"rowref", w.rowref, (size_t)rows * sizeof(float)},
        {"rowlo", w.rowlo, (size_t)rows * sizeof(float)},
        {"fbcnt", w.fbcnt, sizeof(uint32_t)},
        {"fblist", w.fblist, (size_t)rows * sizeof(uint32_t)},
        {"fbsync", w.fbsync, (size_t)FB_GRID * FB_SYNC_WORDS * sizeof(uint32_t)},
        {"fbpart", w.fbpart, (size_t)fb_grid(rows) * FB_PART_BYTES},
    };
    const int nr = (int)(sizeof r / sizeof r[0]);
    for (int i = 0; i < nr; ++i) {
        const char *what = nullptr;
        CHECK(r[i].p != nullptr, "kernel %d: %s is null", kernel, r[i].name);
        if (!r[i].p) continue;
        CHECK(((uintptr_t)r[i].p & 15u) == 0, "kernel %d: %s misaligned", kernel, r[i].name);
        CHECK(inside(r[i].p, r[i].n, &what), "kernel %d: %s (%zu bytes, %d rows) outside the workspace",
              kernel, r[i].name, r[i].n, rows);
        for (int k = 0; k < i; ++k) {
            const char *a = (const char *)r[i].p, *b = (const char *)r[k].p;
            CHECK(a + r[i].n <= b || b + r[k].n <= a, "kernel %d: %s overlaps %s", kernel,
                  r[i].name, r[k].name);
        }
        memset(r[i].p, 0xA5, r[i].n);
    }
}

static hipError_t record(int kernel, const KParams &p, const KPlan &l, const KWork &w, int dtype,
                         bool al) {
    CHECK(p.B >= 1 && p.b0 >= 0 && p.b0 + p.B <= call_batch, "kernel %d rows %d+%d of %d", kernel,
          p.b0, p.B, call_batch);
    const int64_t per_row = kernel == 1 ? l.nt : kernel == 4 ? l.ntd : 1;
    CHECK((int64_t)p.B * per_row <= ((int64_t)1 << 23), "kernel %d grid %lld", kernel,
          (long long)((int64_t)p.B * per_row));
    CHECK(l.nt >= 1 && (int64_t)4 * l.nt * l.wcap <= ROWCAP && l.cus == cus, "plan");
    CHECK(p.V >= 1 && p.V <= SAMPLER_VOCAB_MAX && p.ld >= p.V, "V %d ld %lld", p.V,
          (long long)p.ld);
    touch_workspace(l, w, p.b0 + p.B, kernel);
    launches.push_back({kernel, p.b0, p.B, dtype, al, l});
    return kernel == fail_launch_kernel ? hipErrorLaunchFailure : hipSuccess;
}

namespace smp {
hipError_t launch_plan(const KParams &p, const KPlan &l, const KWork &w, int dtype, bool al,
                       hipStream_t) {
    return record(0, p, l, w, dtype, al);
}
hipError_t launch_pass(const KParams &p, const KPlan &l, const KWork &w, int dtype, bool al,
                       hipStream_t) {
    return record(1, p, l, w, dtype, al);
}
hipError_t launch_rows(const KParams &p, const KPlan &l, const KWork &w, hipStream_t) {
    return record(2, p, l, w, -1, false);
}
hipError_t launch_fallback(const KParams &p, const KPlan &l, const KWork &w, int dtype, bool al,
                           hipStream_t) {
    CHECK(p.b0 == 0 && p.B == call_batch, "fallback spans the whole call");
    return record(3, p, l, w, dtype, al);
}
hipError_t launch_dense(const KParams &p, const KPlan &l, const KWork &w, int dtype, bool al,
                        hipStream_t) {
    return record(4, p, l, w, dtype, al);
}
hipError_t launch_epilogue(const EpiParams &e, hipStream_t) {
    CHECK(e.B == call_batch && e.out_idx != nullptr, "epilogue rows %d", e.B);
    launches.push_back({5, 0, e.B, -1, false, KPlan{}});
    return fail_launch_kernel == 5 ? hipErrorLaunchFailure : hipSuccess;
}
hipError_t static_scratch(int device, void **ptr) {
    CHECK(device == 0, "device %d", device);
    if (static_area.empty()) static_area.resize(SAMPLER_STATIC_SCRATCH_BYTES);
    *ptr = static_area.data();
    return hipSuccess;
}
}  // namespace smp

// ---------------------------------------------------------------------------
// Cases.

struct Bufs {
    std::vector<float> logits, q, u, top_p, out_logits, out_probs;
    std::vector<int32_t> top_k, ids, len, counts;
    std::vector<int64_t> out_idx, offsets;
    std::vector<uint8_t> flags, finished;
    sampler_args a;
    Bufs(int B, int V) {
        logits.assign((size_t)B * V + 4, 0.0f);
        q.assign((size_t)B * V + 4, 1.0f);
        u.assign(B, 0.5f);
        top_p.assign(B, 0.9f);
        top_k.assign(B, 50);
        out_logits.assign((size_t)B * V + 4, 0.0f);
        out_probs.assign((size_t)B * V + 4, 0.0f);
        ids.assign((size_t)B * 4, 1);
        len.assign(B, 2);
        counts.assign(2, 0);
        out_idx.assign(B, 0);
        offsets.resize(B + 1);
        for (int b = 0; b <= B; ++b) offsets[b] = 4 * b;
        flags.assign(B, SAMPLER_ROW_ALL);
        finished.assign(B, 0);
        memset(&a, 0, sizeof a);
        a.logits = logits.data();
        a.ld = V;
        a.top_k = top_k.data();
        a.top_p = top_p.data();
        a.q = q.data();
        a.row_flags = flags.data();
        a.out_idx = out_idx.data();
        a.temperature = 1.0f;
        a.repetition_penalty = 1.0f;
        a.eps = 1e-20f;
    }
};

static std::vector<int> kernels_of(size_t from) {
    std::vector<int> k;
    for (size_t i = from; i < launches.size(); ++i)
        if (k.empty() || k.back() != launches[i].kernel) k.push_back(launches[i].kernel);
    return k;
}

// Rows of each kernel's launches cover [0, batch) once, in order.
static void check_cover(size_t from, int batch) {
    for (int k = 0; k <= 4; ++k) {
        int next = 0;
        bool any = false;
        for (size_t i = from; i < launches.size(); ++i)
            if (launches[i].kernel == k) {
                any = true;
                CHECK(launches[i].b0 == next, "kernel %d chunk at %d, expected %d", k,
                      launches[i].b0, next);
                next = launches[i].b0 + launches[i].B;
            }
        CHECK(!any || next == batch, "kernel %d covers %d of %d rows", k, next, batch);
    }
}

static void argument_checks() {
    sampler_t *h = nullptr;
    CHECK(sampler_create(nullptr, 4, 100, SAMPLER_F32, nullptr) == SAMPLER_EINVAL, "null handle");
    CHECK(sampler_create(&h, 0, 100, SAMPLER_F32, nullptr) == SAMPLER_EINVAL && !h, "batch 0");
    CHECK(sampler_create(&h, 4, 0, SAMPLER_F32, nullptr) == SAMPLER_EINVAL, "vocab 0");
    CHECK(sampler_create(&h, 4, SAMPLER_VOCAB_MAX + 1, SAMPLER_F32, nullptr) == SAMPLER_EINVAL,
          "vocab too large");
    CHECK(sampler_create(&h, 4, 100, 7, nullptr) == SAMPLER_EINVAL, "dtype");
    sampler_opts o;
    memset(&o, 0, sizeof o);
    o.segment_len = 1000;
    CHECK(sampler_create(&h, 4, 100, SAMPLER_F32, &o) == SAMPLER_EINVAL, "segment 1000");
    o.segment_len = SEG_MAX + SEG_MIN;
    CHECK(sampler_create(&h, 4, 100, SAMPLER_F32, &o) == SAMPLER_EINVAL, "segment too long");
    o.segment_len = 0;
    o.topk_guess = SAMPLER_TOPK_MAX + 1;
    CHECK(sampler_create(&h, 4, 100, SAMPLER_F32, &o) == SAMPLER_EINVAL, "guess");
    o.topk_guess = 0;
    o.rows_per_launch = -1;
    CHECK(sampler_create(&h, 4, 100, SAMPLER_F32, &o) == SAMPLER_EINVAL, "rows per launch");

    // runtime failures in create leave nothing allocated
    fail_get_device = 1;
    CHECK(sampler_create(&h, 4, 100, SAMPLER_F32, nullptr) == SAMPLER_EHIP && !h, "get device");
    fail_attribute = 1;
    CHECK(sampler_create(&h, 4, 100, SAMPLER_F32, nullptr) == SAMPLER_EHIP && !h, "attribute");
    fail_malloc = hipErrorOutOfMemory;
    CHECK(sampler_create(&h, 4, 100, SAMPLER_F32, nullptr) == SAMPLER_ENOMEM && !h, "oom");
    fail_malloc = hipErrorInvalidValue;
    CHECK(sampler_create(&h, 4, 100, SAMPLER_F32, nullptr) == SAMPLER_EHIP && !h, "malloc");
    CHECK(live.empty(), "allocations left after failed creates");
    CHECK(sampler_destroy(nullptr) == SAMPLER_OK, "destroy null");
    CHECK(sampler_check(nullptr, 1, nullptr) == SAMPLER_EINVAL, "check null handle");
    CHECK(strcmp(sampler_strerror(SAMPLER_EINVAL), "invalid argument") == 0 &&
              strcmp(sampler_strerror(12345), "unknown error") == 0,
          "strerror");

    const int B = 6, V = 300;
    CHECK(sampler_create(&h, B, V, SAMPLER_F32, nullptr) == SAMPLER_OK && h, "create");
    Bufs f(B, V);
    sampler_args a = f.a;
    CHECK(sampler_check(h, B, &a) == SAMPLER_OK, "valid");
    CHECK(sampler_check(h, B, nullptr) == SAMPLER_EINVAL, "null args");
    CHECK(sampler_check(h, B + 1, &a) == SAMPLER_EINVAL, "batch above max");
    CHECK(sampler_check(h, -1, &a) == SAMPLER_EINVAL, "negative batch");
    CHECK(sampler_run(h, 0, &a, nullptr) == SAMPLER_OK, "empty batch");
    auto bad = [&](const char *what, auto &&edit) {
        sampler_args x = f.a;
        edit(x);
        CHECK(sampler_check(h, B, &x) == SAMPLER_EINVAL, "%s accepted", what);
        const size_t n0 = launches.size();
        CHECK(sampler_run(h, B, &x, nullptr) == SAMPLER_EINVAL, "%s ran", what);
        CHECK(launches.size() == n0, "%s launched", what);
    };
    bad("null logits", [](sampler_args &x) { x.logits = nullptr; });
    bad("null out_idx", [](sampler_args &x) { x.out_idx = nullptr; });
    bad("ld < V", [](sampler_args &x) { x.ld = 299; });
    bad("T = 0", [](sampler_args &x) { x.temperature = 0.0f; });
    bad("T = nan", [](sampler_args &x) { x.temperature = NAN; });
    bad("T = inf", [](sampler_args &x) { x.temperature = INFINITY; });
    bad("rho = 0", [](sampler_args &x) { x.repetition_penalty = 0.0f; });
    bad("rho = nan", [](sampler_args &x) { x.repetition_penalty = NAN; });
    bad("eps < 0", [](sampler_args &x) { x.eps = -1e-20f; });
    bad("eps = inf", [](sampler_args &x) { x.eps = INFINITY; });
    bad("unknown flag", [](sampler_args &x) { x.flags = 1u << 20; });
    bad("logits flag without buffer", [](sampler_args &x) { x.flags = SAMPLER_NEED_LOGITS; });
    bad("probs flag without buffer", [](sampler_args &x) { x.flags = SAMPLER_NEED_PROBS; });
    bad("ids without offsets", [&](sampler_args &x) { x.penalty_ids = f.ids.data(); });
    bad("offsets without ids", [&](sampler_args &x) { x.penalty_offsets = f.offsets.data(); });
    bad("len without ids", [&](sampler_args &x) { x.penalty_len = f.len.data(); });
    bad("append without len", [&](sampler_args &x) {
        x.penalty_ids = f.ids.data();
        x.penalty_offsets = f.offsets.data();
        x.flags = SAMPLER_APPEND_HISTORY;
    });
    bad("finished with eos out of range", [&](sampler_args &x) {
        x.finished = f.finished.data();
        x.eos_id = V;
    });
    bad("no flags, no q, no u", [](sampler_args &x) {
        x.row_flags = nullptr;
        x.q = nullptr;
        x.u = nullptr;
    });
    CHECK(sampler_destroy(h) == SAMPLER_OK && live.empty(), "destroy");
}

// One call through the handle and one through the static entry point, with
// the launch sequence and chunking checked.
static void run_case(int B, int V, int dtype, const sampler_opts *opts, bool filtering, bool u,
                     uint32_t flags, bool epilogue, int expect_chunk) {
    sampler_t *h = nullptr;
    CHECK(sampler_create(&h, B, V, dtype, opts) == SAMPLER_OK, "create B=%d V=%d", B, V);
    if (!h) return;
    Bufs f(B, V);
    sampler_args a = f.a;
    if (!filtering) {
        a.top_k = nullptr;
        a.top_p = nullptr;
    }
    if (u) {
        a.u = f.u.data();
        a.q = nullptr;
    }
    a.flags = flags;
    if (flags & SAMPLER_NEED_LOGITS) a.out_logits = f.out_logits.data();
    if (flags & SAMPLER_NEED_PROBS) a.out_probs = f.out_probs.data();
    if (epilogue) {
        a.penalty_ids = f.ids.data();
        a.penalty_offsets = f.offsets.data();
        a.penalty_len = f.len.data();
        a.finished = f.finished.data();
        a.eos_id = 0;
        a.counts = f.counts.data();
        a.flags |= SAMPLER_APPEND_HISTORY;
        a.repetition_penalty = 1.3f;
    }
    for (int path = 0; path < 2; ++path) {
        if (path == 1 && (a.flags & SAMPLER_PROFILE)) break;
        call_batch = B;
        const size_t n0 = launches.size();
        int rc;
        if (path == 0) {
            rc = sampler_run(h, B, &a, nullptr);
        } else {
            rc = sampler_run_static(B, V, dtype, opts, &a, nullptr);
            if (rc == SAMPLER_EINVAL) {
                // only when the workspace of B rows exceeds the static area
                const KPlan l = make_plan(V, opts && opts->segment_len ? opts->segment_len
                                                                       : auto_seg(B, V, cus),
                                          cus);
                CHECK((size_t)B * ROWCAP * 8 > (size_t)SAMPLER_STATIC_SCRATCH_BYTES / 2 ||
                          l.nt > 64,
                      "static path refused B=%d V=%d", B, V);
                continue;
            }
        }
        CHECK(rc == SAMPLER_OK, "run path %d B=%d V=%d rc=%d", path, B, V, rc);
        std::vector<int> ks = kernels_of(n0);
        std::vector<int> want;
        if (filtering) want.push_back(0);
        want.push_back(1);
        want.push_back(2);
        if (filtering || u) want.push_back(3);
        if ((flags & SAMPLER_NEED_PROBS) || ((flags & SAMPLER_NEED_LOGITS) && filtering))
            want.push_back(4);
        if (epilogue) want.push_back(5);
        CHECK(ks == want, "path %d B=%d V=%d: kernel sequence differs (%zu vs %zu kernels)", path,
              B, V, ks.size(), want.size());
        check_cover(n0, B);
        for (size_t i = n0; i < launches.size(); ++i) {
            const Launch &L = launches[i];
            if (L.kernel == 1 || L.kernel == 4)
                CHECK(expect_chunk <= 0 || L.B <= expect_chunk, "chunk of %d rows > %d", L.B,
                      expect_chunk);
            if (L.kernel != 2 && L.kernel != 5)
                CHECK(L.dtype == dtype, "dtype %d", L.dtype);
        }
    }
    if (flags & SAMPLER_PROFILE) {
        float ms[SAMPLER_PROFILE_SLOTS + 2];
        const int n = sampler_profile(h, ms, SAMPLER_PROFILE_SLOTS + 2);
        CHECK(n == SAMPLER_PROFILE_SLOTS, "profile slots %d", n);
        CHECK(sampler_profile(h, ms, 4) == SAMPLER_EINVAL, "profile read twice");
    }
    CHECK(sampler_destroy(h) == SAMPLER_OK, "destroy");
    CHECK(live.empty(), "leak B=%d V=%d", B, V);
    CHECK(n_events_live == 0, "events left");
}

static void launch_failures() {
    const int B = 5, V = 5000;
    for (int k = 0; k <= 5; ++k) {
        sampler_t *h = nullptr;
        CHECK(sampler_create(&h, B, V, SAMPLER_BF16, nullptr) == SAMPLER_OK, "create");
        Bufs f(B, V);
        sampler_args a = f.a;
        a.u = f.u.data();
        a.out_probs = f.out_probs.data();
        a.flags = SAMPLER_NEED_PROBS;
        a.finished = f.finished.data();
        call_batch = B;
        fail_launch_kernel = k;
        const size_t n0 = launches.size();
        CHECK(sampler_run(h, B, &a, nullptr) == SAMPLER_EHIP, "launch %d failure not reported", k);
        CHECK(launches.back().kernel == k, "kernels ran after the failed launch %d", k);
        fail_launch_kernel = -1;
        (void)n0;
        CHECK(sampler_run(h, B, &a, nullptr) == SAMPLER_OK, "run after a failed launch");
        sampler_destroy(h);
    }
    // profiling when events cannot be made: the call still runs, unprofiled
    sampler_t *h = nullptr;
    CHECK(sampler_create(&h, 2, 100, SAMPLER_F32, nullptr) == SAMPLER_OK, "create");
    Bufs f(2, 100);
    sampler_args a = f.a;
    a.flags = SAMPLER_PROFILE;
    call_batch = 2;
    fail_event_create = 5;
    CHECK(sampler_run(h, 2, &a, nullptr) == SAMPLER_OK, "run without events");
    fail_event_create = 0;
    float ms[8];
    CHECK(sampler_profile(h, ms, 8) == SAMPLER_EINVAL, "profile without events");
    CHECK(sampler_profile(nullptr, ms, 8) == SAMPLER_EINVAL && sampler_profile(h, nullptr, 8) ==
              SAMPLER_EINVAL, "profile arguments");
    sampler_destroy(h);
    CHECK(n_events_live == 0 && live.empty(), "events or blocks left");
    // the static entry point: profiling, sizes and batch limits
    call_batch = 2;
    a.flags = SAMPLER_PROFILE;
    CHECK(sampler_run_static(2, 100, SAMPLER_F32, nullptr, &a, nullptr) == SAMPLER_EINVAL,
          "static profile");
    a.flags = 0;
    CHECK(sampler_run_static(-1, 100, SAMPLER_F32, nullptr, &a, nullptr) == SAMPLER_EINVAL,
          "static negative batch");
    CHECK(sampler_run_static(0, 100, SAMPLER_F32, nullptr, &a, nullptr) == SAMPLER_OK,
          "static empty batch");
    CHECK(sampler_run_static(2, 0, SAMPLER_F32, nullptr, &a, nullptr) == SAMPLER_EINVAL,
          "static vocab 0");
    // 8192 rows need 8192 * ROWCAP * 8 bytes of candidates alone: above the area
    Bufs big(1, 100);
    sampler_args ab = big.a;
    ab.top_k = nullptr;
    ab.top_p = nullptr;
    ab.row_flags = nullptr;
    ab.q = nullptr;
    ab.u = nullptr;
    ab.row_flags = big.flags.data();
    CHECK(sampler_run_static(8192, 100, SAMPLER_F32, nullptr, &ab, nullptr) == SAMPLER_EINVAL,
          "static workspace above the limit");
}

int main() {
    argument_checks();
    sampler_opts o;
    memset(&o, 0, sizeof o);
    // small and ragged shapes, both dtypes, every output combination
    const int shapes[][2] = {{1, 1}, {1, 7}, {3, 2047}, {4, 2048}, {5, 2049}, {2, 8191},
                             {7, 8193}, {3, 50257}, {2, 262144}, {1, SAMPLER_VOCAB_MAX}};
    for (auto &s : shapes)
        for (int dtype = 0; dtype < 2; ++dtype)
            for (int mode = 0; mode < 6; ++mode) {
                const bool filt = mode != 1 && mode != 4;
                const bool u = mode == 2 || mode == 4;
                const uint32_t fl = mode == 3 ? SAMPLER_NEED_LOGITS | SAMPLER_NEED_PROBS
                                  : mode == 4 ? SAMPLER_NEED_LOGITS
                                  : mode == 5 ? SAMPLER_NEED_LOGITS | SAMPLER_PROFILE
                                              : 0u;
                run_case(s[0], s[1], dtype, nullptr, filt, u, fl, mode == 2, 0);
            }
    // tile lengths, and rows split over several launches
    for (int seg = SEG_MIN; seg <= SEG_MAX; seg *= 2) {
        o.segment_len = seg;
        o.rows_per_launch = 3;
        run_case(10, 70001, SAMPLER_BF16, &o, true, false, SAMPLER_NEED_PROBS, true, 3);
    }
    o.segment_len = 0;
    o.rows_per_launch = 0;
    run_case(64, 262144, SAMPLER_F32, &o, true, false, SAMPLER_NEED_LOGITS, false, 0);
    launch_failures();
    if (failures) {
        fprintf(stderr, "%d failed checks\n", failures);
        return 1;
    }
    printf("api checks ok: %zu launches recorded\n", launches.size());
    return 0;
}
