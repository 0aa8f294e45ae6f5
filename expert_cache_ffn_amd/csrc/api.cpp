// C-ABI entry points of libecf: errors, layouts, workspace, prefetch, profiling
// hooks and the layer forward (all-resident and expert-cache modes).
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "cache_internal.h"
#include "ecf_internal.h"
#include "host_ffn.h"

namespace ecf {

// ---- errors ----------------------------------------------------------------------
static thread_local std::string g_err;

int set_error(int code, const char *fmt, ...)
{
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

// ---- profiling ---------------------------------------------------------------------
namespace {
struct ProfAcc {
    std::string name;
    int64_t n = 0;
    double ms = 0.0;
};
struct Pending {
    int idx;
    hipEvent_t a, b;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};  // read by every launch, on any thread
std::vector<ProfAcc> g_prof;
std::vector<Pending> g_pending;

int prof_index(const char *name)
{
    for (size_t i = 0; i < g_prof.size(); ++i)
        if (g_prof[i].name == name)
            return (int)i;
    g_prof.push_back(ProfAcc{name});
    return (int)g_prof.size() - 1;
}

int prof_resolve()
{
    std::lock_guard<std::mutex> g(g_prof_mu);
    if (g_pending.empty())
        return ECF_OK;
    ECF_HIP_CHECK(hipDeviceSynchronize());
    for (auto &p : g_pending) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
            g_prof[p.idx].n += 1;
            g_prof[p.idx].ms += ms;
        }
        (void)hipEventDestroy(p.a);
        (void)hipEventDestroy(p.b);
    }
    g_pending.clear();
    return ECF_OK;
}
}  // namespace

thread_local bool t_prof_quiet = false;

ProfScope::ProfScope(const char *name, hipStream_t s) : name_(name), s_(s)
{
    if (!g_prof_on || t_prof_quiet)
        return;
    if (hipEventCreate(&a_) != hipSuccess) {
        a_ = nullptr;
        return;
    }
    if (hipEventCreate(&b_) != hipSuccess) {
        (void)hipEventDestroy(a_);
        a_ = b_ = nullptr;
        return;
    }
    (void)hipEventRecord(a_, s_);
}

ProfScope::~ProfScope()
{
    if (!a_)
        return;
    (void)hipEventRecord(b_, s_);
    std::lock_guard<std::mutex> g(g_prof_mu);
    g_pending.push_back(Pending{prof_index(name_), a_, b_});
}

// ---- layouts -------------------------------------------------------------------------
static inline size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

static int check_shape(const ecf_shape *s)
{
    if (!s)
        return set_error(ECF_EINVAL, "shape is NULL");
    if (s->hidden <= 0 || s->hidden % 256 || s->inter <= 0 || s->inter % 64)
        return set_error(ECF_EINVAL, "hidden must be a positive multiple of 256 and inter of 64 (d=%d, I=%d)",
                         s->hidden, s->inter);
    if (s->n_experts < 1 || s->n_experts > 1024 || s->top_k < 1 || s->top_k > 32 || s->top_k > s->n_experts)
        return set_error(ECF_EINVAL, "need 1 <= E <= 1024 and 1 <= k <= min(E, 32) (E=%d, k=%d)",
                         s->n_experts, s->top_k);
    if (s->w_dtype < ECF_F32 || s->w_dtype > ECF_MXFP4 || (s->a_dtype != ECF_F32 && s->a_dtype != ECF_BF16))
        return set_error(ECF_EINVAL, "bad dtype (w=%d, a=%d)", s->w_dtype, s->a_dtype);
    if (s->w_dtype != ECF_F32 && s->a_dtype != ECF_BF16)
        return set_error(ECF_EINVAL, "bf16 or MXFP4 weights need bf16 activations");
    if (s->renorm_topk != 0 && s->renorm_topk != 1)
        return set_error(ECF_EINVAL, "renorm_topk must be 0 or 1");
    return ECF_OK;
}

bool blob_layout(const ecf_shape &s, BlobLayout *out)
{
    const size_t n = (size_t)s.hidden * s.inter;
    size_t mat;
    if (s.w_dtype == ECF_F32)
        mat = n * 4;
    else if (s.w_dtype == ECF_BF16)
        mat = n * 2;
    else
        mat = n / 2;
    out->off[0] = 0;
    out->off[1] = al256(mat);
    out->off[2] = out->off[1] + al256(mat);
    size_t end = out->off[2] + al256(mat);
    if (s.w_dtype == ECF_MXFP4) {
        const size_t sc = n / 32;
        out->off[3] = end;
        out->off[4] = end + al256(sc);
        out->off[5] = out->off[4] + al256(sc);
        end = out->off[5] + al256(sc);
    } else {
        out->off[3] = out->off[4] = out->off[5] = 0;
    }
    out->bytes = end;
    return true;
}

int max_tiles(const ecf_shape &s, int32_t T)
{
    const int R = T * s.top_k;
    const int mt = prefill_mt(s);
    return (R + mt - 1) / mt + std::min(s.n_experts, R);
}

WsLayout ws_layout(const ecf_shape &s, int32_t T)
{
    const size_t R = (size_t)T * s.top_k, E = s.n_experts, d = s.hidden, I = s.inter;
    const size_t S = (R + kSortSeg - 1) / kSortSeg;
    WsLayout w{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += al256(std::max<size_t>(bytes, 1));
        return at;
    };
    w.logits = take(4 * (size_t)T * E);
    w.idx = take(4 * R);
    w.gate = take(4 * R);
    w.counts = take(4 * E);
    w.offsets = take(4 * (E + 1));
    w.perm = take(4 * R);
    w.pos = take(4 * R);
    w.active = take(4 * E);
    w.n_active = take(4);
    w.tiles = take(8 * (size_t)max_tiles(s, T));
    w.n_tiles = take(4);
    w.seg_counts = take(4 * S * E);
    w.seg_base = take(4 * S * E);
    w.ptrs = take(3 * 8 * E);  // cache mode: hits, copied misses, both
    w.hbuf = take(4 * R * I);
    w.ybuf = take(4 * R * d);
    w.host_out = take(4 * (size_t)T * d);
    w.total = o;
    return w;
}

// ---- cache host resources ------------------------------------------------------------
int staging(ecf_cache::Staging &s, size_t bytes)
{
    if (s.bytes >= bytes)
        return ECF_OK;
    if (s.p)
        (void)hipHostFree(s.p);
    s.p = nullptr;
    s.bytes = 0;
    const size_t want = std::max<size_t>(bytes, 4096);
    ECF_HIP_CHECK(hipHostMalloc(&s.p, want, hipHostMallocDefault));
    s.bytes = want;
    return ECF_OK;
}

void cache_release_host(ecf_cache *c)
{
    // pending prefetch copies still write into the caller's slot memory
    while (!c->prefetched.empty()) {
        hipEvent_t ev = cache_take_prefetch(c, c->prefetched.front().layer);
        if (ev) {
            (void)hipEventSynchronize(ev);
            (void)hipEventDestroy(ev);
        }
    }
    for (hipEvent_t ev : c->spare_events)
        (void)hipEventDestroy(ev);
    c->spare_events.clear();
    if (c->last_compute)
        (void)hipEventDestroy(c->last_compute);
    for (auto *s : {&c->st_counts, &c->st_idx, &c->st_gate, &c->st_x, &c->st_out, &c->st_ptrs, &c->st_y})
        if (s->p)
            (void)hipHostFree(s->p);
    if (c->copy_done)
        (void)hipEventDestroy(c->copy_done);
    delete c->pool;
    c->pool = nullptr;
}

}  // namespace ecf

using namespace ecf;

// ---------------------------------------------------------------------------------------
extern "C" {

const char *ecf_last_error(void) { return g_err.c_str(); }

size_t ecf_expert_bytes(const ecf_shape *shape)
{
    if (check_shape(shape) != ECF_OK)
        return 0;
    BlobLayout l;
    blob_layout(*shape, &l);
    return l.bytes;
}

int ecf_expert_layout(const ecf_shape *shape, size_t offsets_out[6])
{
    const int rc = check_shape(shape);
    if (rc != ECF_OK)
        return rc;
    if (!offsets_out)
        return set_error(ECF_EINVAL, "offsets_out is NULL");
    BlobLayout l;
    blob_layout(*shape, &l);
    std::memcpy(offsets_out, l.off, sizeof l.off);
    return ECF_OK;
}

size_t ecf_workspace_bytes(const ecf_shape *shape, int32_t max_tokens)
{
    if (check_shape(shape) != ECF_OK || max_tokens < 0 || (int64_t)max_tokens * shape->top_k > kMaxRows)
        return 0;
    return ws_layout(*shape, max_tokens).total;
}

int prefetch_layer(ecf_cache *c, int32_t layer, size_t blob_bytes, void *copy_stream, void *done_event,
                   int32_t *n_copied, int32_t *n_missing)
{
    return ::ecf::guarded("prefetch_layer", [&]() -> int {
        if (n_copied)
            *n_copied = 0;
        if (n_missing)
            *n_missing = 0;
        if (!c || layer < 0 || layer >= c->L)
            return set_error(ECF_EINVAL, "prefetch_layer: bad cache or layer");
        if (c->h_pool.empty())
            return set_error(ECF_EINVAL, "prefetch_layer: the cache has no host pool");
        if (blob_bytes == 0 || blob_bytes > c->slot_bytes)
            return set_error(ECF_EINVAL, "prefetch_layer: blob_bytes %zu not in [1, slot bytes %zu]", blob_bytes,
                             c->slot_bytes);
        hipStream_t cs = (hipStream_t)copy_stream;
        for (const auto &p : c->prefetched)
            if (p.layer == layer) {  // already pending: nothing to add
                if (n_missing)
                    *n_missing = p.missing;
                if (done_event)
                    ECF_HIP_CHECK(hipEventRecord((hipEvent_t)done_event, cs));
                return ECF_OK;
            }
        hipEvent_t ev = nullptr;
        if (!c->spare_events.empty()) {
            ev = c->spare_events.back();
            c->spare_events.pop_back();
        } else {
            ECF_HIP_CHECK(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
        }
        const int E = c->E;
        c->prefetched.emplace_back();
        ecf_cache::Prefetch &pf = c->prefetched.back();
        pf.layer = layer;
        pf.done = ev;
        // hold the layer's resident entries first, so no bind below evicts them
        for (int e = 0; e < E; ++e) {
            const int32_t sl = c->slot_of[(size_t)layer * E + e];
            if (sl >= 0) {
                c->held[sl] = 1;
                pf.slots.push_back(sl);
            }
        }
        int32_t budget = cache_available(c) - c->reserve;
        // ascending expert id: a resident entry is touched (most recent), a
        // missing one is bound while the budget lasts
        std::vector<int32_t> bexp, bslot;
        bool evicted = false;
        int32_t missing = 0;
        for (int e = 0; e < E; ++e) {
            const int32_t sl = c->slot_of[(size_t)layer * E + e];
            if (sl >= 0) {
                cache_touch(c, sl);
                continue;
            }
            if (budget <= 0) {
                ++missing;
                continue;
            }
            int32_t victim = -1;
            const int32_t ns = cache_bind(c, layer, e, &victim);
            if (ns < 0) {  // cannot happen: the budget counts bindable slots
                ++missing;
                continue;
            }
            --budget;
            evicted |= victim >= 0;
            c->held[ns] = 1;
            pf.slots.push_back(ns);
            bexp.push_back(e);
            bslot.push_back(ns);
        }
        pf.missing = missing;
        c->reserve += missing;
        // a slot taken from another entry may still be read by queued kernels
        if (evicted && c->have_last_compute)
            ECF_HIP_CHECK(hipStreamWaitEvent(cs, c->last_compute, 0));
        {
            ProfScope p("prefetch_layer_copy", cs);
            // runs of consecutive slots fed by consecutive host blobs go as one copy
            const bool packed = blob_bytes == c->slot_bytes;
            for (size_t i = 0; i < bexp.size();) {
                size_t j = i + 1;
                const char *h0 = (const char *)c->h_pool[(size_t)layer * E + bexp[i]];
                while (packed && j < bexp.size() && bslot[j] == bslot[j - 1] + 1 &&
                       (const char *)c->h_pool[(size_t)layer * E + bexp[j]] == h0 + (j - i) * blob_bytes)
                    ++j;
                const size_t bytes = (j - i - 1) * c->slot_bytes + blob_bytes;
                ECF_HIP_CHECK(hipMemcpyAsync(c->d_slots + (size_t)bslot[i] * c->slot_bytes, h0, bytes,
                                             hipMemcpyHostToDevice, cs));
                i = j;
            }
        }
        ECF_HIP_CHECK(hipEventRecord(ev, cs));
        if (done_event)
            ECF_HIP_CHECK(hipEventRecord((hipEvent_t)done_event, cs));
        if (n_copied)
            *n_copied = (int32_t)bexp.size();
        if (n_missing)
            *n_missing = missing;
        return ECF_OK;
    });
}

int ecf_host_experts(const ecf_shape *shape, int32_t n_jobs, const void *const *h_blobs,
                     const int32_t *n_rows, const int32_t *rows, const void *h_x, int32_t n_tokens,
                     float *h_y, int32_t n_threads)
{
    try {
        int rc = check_shape(shape);
        if (rc != ECF_OK)
            return rc;
        if (n_jobs < 0 || n_tokens < 0 || n_threads < 0 || (int64_t)n_tokens * shape->top_k > kMaxRows ||
            (n_jobs > 0 && (!h_blobs || !n_rows || !rows || !h_x || !h_y)))
            return set_error(ECF_EINVAL, "ecf_host_experts: bad arguments");
        BlobLayout lay;
        blob_layout(*shape, &lay);
        std::vector<HostExpertJob> jobs(n_jobs);
        const int R = n_tokens * shape->top_k;
        int at = 0;
        for (int32_t i = 0; i < n_jobs; ++i) {
            jobs[i].expert = i;
            jobs[i].blob = h_blobs[i];
            if (n_rows[i] < 0)
                return set_error(ECF_EINVAL, "ecf_host_experts: negative row count");
            for (int32_t r = 0; r < n_rows[i]; ++r, ++at) {
                if (rows[at] < 0 || rows[at] >= R)
                    return set_error(ECF_EINVAL, "ecf_host_experts: row %d out of range", rows[at]);
                jobs[i].rows.push_back(rows[at]);
            }
        }
        const int nt = n_threads > 0 ? n_threads
                                     : (int)std::min(16u, std::max(1u, std::thread::hardware_concurrency()));
        HostPool pool(nt);
        return host_experts(pool, *shape, lay, jobs, h_x, n_tokens, h_y);
    } catch (...) {
        return set_error(ECF_EINVAL, "ecf_host_experts: failure");
    }
}

int ecf_profile_enable(int32_t on)
{
    return ::ecf::guarded("ecf_profile_enable", [&]() -> int {
        std::lock_guard<std::mutex> g(g_prof_mu);
        g_prof_on = on != 0;
        return ECF_OK;
    });
}

int ecf_profile_get(int32_t i, const char **name, int64_t *launches, double *total_ms)
{
    return ::ecf::guarded("ecf_profile_get", [&]() -> int {
        const int rc = prof_resolve();
        if (rc != ECF_OK)
            return rc;
        std::lock_guard<std::mutex> g(g_prof_mu);
        if (i < 0 || i >= (int32_t)g_prof.size())
            return set_error(ECF_EINVAL, "ecf_profile_get: no entry %d", i);
        if (name)
            *name = g_prof[i].name.c_str();
        if (launches)
            *launches = g_prof[i].n;
        if (total_ms)
            *total_ms = g_prof[i].ms;
        return ECF_OK;
    });
}

int ecf_profile_reset(void)
{
    return ::ecf::guarded("ecf_profile_reset", [&]() -> int {
        const int rc = prof_resolve();
        std::lock_guard<std::mutex> g(g_prof_mu);
        g_prof.clear();
        return rc;
    });
}

// ---------------------------------------------------------------------------------------

static int pick_path(const ecf_layer_args *a, int32_t T)
{
    if (a->path == ECF_PATH_DECODE || a->path == ECF_PATH_PREFILL)
        return a->path;
    // Cache mode: the decode GEMVs keep h in fp32 like the host experts, so the
    // output does not depend on the split (the prefill GEMM rounds h to bf16).
    if (a->cache || a->shape.w_dtype == ECF_F32)
        return ECF_PATH_DECODE;
    // bf16 and MXFP4: GEMV while each expert sees a few rows, grouped GEMM beyond
    return (T <= 64 || a->shape.inter % 128) ? ECF_PATH_DECODE : ECF_PATH_PREFILL;
}

// The expert kernels of one layer on the experts `ex` lists (0 = skipped).
static int launch_experts(const ecf_shape &s, const ExpertTables &ex, const RouteOut &ro, const void *d_x,
                          int32_t T, const WsLayout &wl, char *ws, int path, hipStream_t stream)
{
    int rc;
    if (path == ECF_PATH_DECODE) {
        if ((rc = launch_decode_gateup(s, ex, ro, d_x, T, (float *)(ws + wl.hbuf), stream)) ||
            (rc = launch_decode_down(s, ex, ro, (const float *)(ws + wl.hbuf), T, (float *)(ws + wl.ybuf),
                                     stream)))
            return rc;
    } else {
        if ((rc = launch_prefill_gemm1(s, ex, ro, d_x, T, (uint16_t *)(ws + wl.hbuf), stream)) ||
            (rc = launch_prefill_gemm2(s, ex, ro, (const uint16_t *)(ws + wl.hbuf), T, (float *)(ws + wl.ybuf),
                                       stream)))
            return rc;
    }
    return ECF_OK;
}

// Expert-cache placement for one layer-step: read the routing back, look the
// step's experts up, split the misses by q*, bind and fill slots for the
// copied ones, and queue the GPU work -- the hits' kernels first, the copied
// experts' kernels once their copies have landed; the host-assigned experts
// are then evaluated on the cache's threads and their partial sum is queued
// for the combine.  On the prefill path every miss is copied (the grouped
// GEMM rounds h to bf16, the host experts do not, so a split would make the
// output depend on it).  Writes the combine's expert table (hits and copied
// misses) and the device address of the host partial (or NULL).
static int cache_step(const ecf_layer_args *a, const void *d_x, int32_t T, const RouteOut &ro,
                      const WsLayout &wl, char *ws, const BlobLayout &lay, int path, ecf_step_stats *st,
                      const uint64_t **gpu_table, const float **host_part_out)
{
    ecf_cache *c = a->cache;
    const ecf_shape &s = a->shape;
    const int E = s.n_experts, k = s.top_k, d = s.hidden, R = T * k;
    hipStream_t stream = (hipStream_t)a->stream;
    hipStream_t cstream = a->copy_stream ? (hipStream_t)a->copy_stream : stream;
    *host_part_out = nullptr;
    if (a->layer < 0 || a->layer >= c->L || c->E != E)
        return set_error(ECF_EINVAL, "cache mode: layer %d / E %d do not match the cache", a->layer, E);
    if (c->h_pool.empty())
        return set_error(ECF_EINVAL, "cache mode needs the cache's host pool");
    if (c->n_slots > 0 && c->slot_bytes < lay.bytes)
        return set_error(ECF_EINVAL, "cache slots (%zu B) smaller than an expert blob (%zu B)", c->slot_bytes,
                         lay.bytes);
    const size_t abytes = (s.a_dtype == ECF_BF16 ? 2 : 4);
    int rc;
    if ((rc = staging(c->st_counts, 4 * (size_t)E)) || (rc = staging(c->st_idx, 4 * (size_t)R)) ||
        (rc = staging(c->st_gate, 4 * (size_t)R)) || (rc = staging(c->st_x, abytes * (size_t)T * d)) ||
        (rc = staging(c->st_out, 4 * (size_t)T * d)) || (rc = staging(c->st_ptrs, 3 * 8 * (size_t)E)) ||
        (rc = staging(c->st_y, 4 * (size_t)R * d)))
        return rc;
    if (!c->copy_done)
        ECF_HIP_CHECK(hipEventCreateWithFlags(&c->copy_done, hipEventDisableTiming));
    if (!c->last_compute)
        ECF_HIP_CHECK(hipEventCreateWithFlags(&c->last_compute, hipEventDisableTiming));
    if (!c->pool) {
        int n = c->host_threads > 0 ? c->host_threads : (int)std::min(16u, std::max(1u, std::thread::hardware_concurrency()));
        c->pool = new HostPool(n);
    }
    // a pending whole-layer prefetch of this layer: its hold ends here, and its
    // copies must land before any kernel reads the layer's slots
    struct PrefetchWait {
        ecf_cache *c;
        hipEvent_t ev;
        ~PrefetchWait() { cache_spare_event(c, ev); }
    } pf{c, cache_take_prefetch(c, a->layer)};
    int32_t *h_counts = (int32_t *)c->st_counts.p, *h_idx = (int32_t *)c->st_idx.p;
    float *h_gate = (float *)c->st_gate.p;
    ECF_HIP_CHECK(hipMemcpyAsync(h_counts, ro.counts, 4 * (size_t)E, hipMemcpyDeviceToHost, stream));
    ECF_HIP_CHECK(hipMemcpyAsync(h_idx, ro.idx, 4 * (size_t)R, hipMemcpyDeviceToHost, stream));
    ECF_HIP_CHECK(hipMemcpyAsync(h_gate, ro.gate, 4 * (size_t)R, hipMemcpyDeviceToHost, stream));
    if (path == ECF_PATH_DECODE)
        ECF_HIP_CHECK(hipMemcpyAsync(c->st_x.p, d_x, abytes * (size_t)T * d, hipMemcpyDeviceToHost, stream));
    const auto t0 = std::chrono::steady_clock::now();
    ECF_HIP_CHECK(hipStreamSynchronize(stream));
    const auto t1 = std::chrono::steady_clock::now();

    std::vector<int32_t> U;
    for (int e = 0; e < E; ++e)
        if (h_counts[e] > 0)
            U.push_back(e);
    std::vector<int32_t> slots(U.size());
    if ((rc = expert_cache_lookup(c, a->layer, U.data(), (int32_t)U.size(), slots.data())) != ECF_OK)
        return rc;
    std::vector<int32_t> miss;
    for (size_t i = 0; i < U.size(); ++i)
        if (slots[i] < 0)
            miss.push_back(U[i]);
    const int32_t m = (int32_t)miss.size();
    int32_t q;
    if (path == ECF_PATH_PREFILL) {
        q = m;
        if (q > ecf_cache_available(c))
            return set_error(ECF_ENOSPC,
                             "cache mode, prefill path: %d missed experts to copy, %d slots available", q,
                             ecf_cache_available(c));
    } else {
        switch (a->q_mode) {
        case ECF_Q_ALL_GPU: q = m; break;
        case ECF_Q_ALL_HOST: q = 0; break;
        case ECF_Q_FIXED: q = std::min(std::max(a->q_fixed, 0), m); break;
        default:
            q = qstar_split(m, a->b_p, a->b_h);
            if (q < 0)
                return q;
        }
        q = std::min(q, ecf_cache_available(c));
    }
    // misses to copy first: most routed rows, then lower id
    std::stable_sort(miss.begin(), miss.end(),
                     [&](int32_t x, int32_t y) { return h_counts[x] > h_counts[y]; });
    std::vector<int32_t> copy_slots(q);
    if ((rc = expert_cache_evict(c, a->layer, miss.data(), q, copy_slots.data(), nullptr)) != ECF_OK)
        return rc;

    // three expert tables: hits, copied misses, and both (for the combine)
    uint64_t *h_hit = (uint64_t *)c->st_ptrs.p, *h_cp = h_hit + E, *h_all = h_cp + E;
    std::memset(h_hit, 0, 3 * 8 * (size_t)E);
    for (size_t i = 0; i < U.size(); ++i)
        if (slots[i] >= 0)
            h_all[U[i]] = h_hit[U[i]] = (uint64_t)(c->d_slots + (size_t)slots[i] * c->slot_bytes);
    int64_t bytes_h2d = 0;
    for (int32_t i = 0; i < q; ++i) {
        char *dst = c->d_slots + (size_t)copy_slots[i] * c->slot_bytes;
        h_all[miss[i]] = h_cp[miss[i]] = (uint64_t)dst;
        const void *src = c->h_pool[(size_t)a->layer * E + miss[i]];
        ProfScope p("slot_fill_copy", cstream);
        ECF_HIP_CHECK(hipMemcpyAsync(dst, src, lay.bytes, hipMemcpyHostToDevice, cstream));
        bytes_h2d += (int64_t)lay.bytes;
    }
    uint64_t *d_tabs = (uint64_t *)(ws + wl.ptrs);  // [3][E]
    ECF_HIP_CHECK(hipMemcpyAsync(d_tabs, h_hit, 3 * 8 * (size_t)E, hipMemcpyHostToDevice, stream));
    if (pf.ev)
        ECF_HIP_CHECK(hipStreamWaitEvent(stream, pf.ev, 0));
    const bool split_launch = q > 0 && cstream != stream && (int32_t)U.size() > m;
    if (split_launch) {  // the hits' kernels run while the copies are in flight
        if ((rc = launch_experts(s, ExpertTables{d_tabs, lay}, ro, d_x, T, wl, ws, path, stream)) != ECF_OK)
            return rc;
    }
    if (q > 0 && cstream != stream) {
        ECF_HIP_CHECK(hipEventRecord(c->copy_done, cstream));
        ECF_HIP_CHECK(hipStreamWaitEvent(stream, c->copy_done, 0));
    }
    const uint64_t *tab = split_launch ? d_tabs + E : d_tabs + 2 * E;
    if ((rc = launch_experts(s, ExpertTables{tab, lay}, ro, d_x, T, wl, ws, path, stream)) != ECF_OK)
        return rc;
    // no later copy may overwrite a slot these kernels read until they are done
    ECF_HIP_CHECK(hipEventRecord(c->last_compute, stream));
    c->have_last_compute = true;
    *gpu_table = d_tabs + 2 * E;
    // the forward call's layer-step ends here: its pins are released
    ++c->gen;
    c->n_pinned = 0;
    c->step_layer = -1;

    // host experts (the m - q misses not copied), in parallel with the GPU
    std::vector<HostExpertJob> jobs;
    int64_t bytes_host = 0;
    for (int32_t i = q; i < m; ++i) {
        HostExpertJob jb;
        jb.expert = miss[i];
        jb.blob = c->h_pool[(size_t)a->layer * E + miss[i]];
        for (int f = 0; f < R; ++f)
            if (h_idx[f] == miss[i])
                jb.rows.push_back(f);
        jobs.push_back(std::move(jb));
        bytes_host += (int64_t)lay.bytes;
    }
    double ms_host = 0.0;
    if (!jobs.empty()) {
        const auto h0 = std::chrono::steady_clock::now();
        float *y = (float *)c->st_y.p;
        if ((rc = host_experts(*c->pool, s, lay, jobs, c->st_x.p, T, y)) != ECF_OK)
            return rc;
        // host partial: per token, host experts in ascending j, gate-weighted
        std::vector<char> is_host(E, 0);
        for (auto &jb : jobs)
            is_host[jb.expert] = 1;
        float *hp = (float *)c->st_out.p;
        c->pool->parallel_for(T, [&](int t) {
            float *o = hp + (size_t)t * d;
            std::fill(o, o + d, 0.f);
            for (int j = 0; j < k; ++j) {
                const int f = t * k + j;
                if (!is_host[h_idx[f]])
                    continue;
                const float g = h_gate[f];
                const float *yy = y + (size_t)f * d;
                for (int cc = 0; cc < d; ++cc)
                    o[cc] = std::fma(g, yy[cc], o[cc]);
            }
        });
        ms_host = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - h0).count();
        float *d_hp = (float *)(ws + wl.host_out);
        ECF_HIP_CHECK(hipMemcpyAsync(d_hp, hp, 4 * (size_t)T * d, hipMemcpyHostToDevice, stream));
        *host_part_out = d_hp;
    }
    if (st) {
        st->n_unique = (int32_t)U.size();
        st->hits = (int32_t)U.size() - m;
        st->misses = m;
        st->q = q;
        st->host = m - q;
        st->bytes_h2d = bytes_h2d;
        st->bytes_host = bytes_host;
        st->ms_wait_route = std::chrono::duration<double, std::milli>(t1 - t0).count();
        st->ms_host_ffn = ms_host;
    }
    return ECF_OK;
}

}  // extern "C"

namespace ecf {

// The forward call with its workspace given explicitly (ws, ws_bytes): the
// caller's buffer for moe_layer_forward, the library's own device array for
// moe_layer_forward_noalloc.
int forward_impl(const ecf_layer_args *a, const void *d_x, int32_t T, float *d_out, ecf_step_stats *stats,
                 void *d_ws, size_t ws_bytes)
{
    try {
        if (!a)
            return set_error(ECF_EINVAL, "moe_layer_forward: NULL args");
        int rc = check_shape(&a->shape);
        if (rc != ECF_OK)
            return rc;
        const ecf_shape &s = a->shape;
        if (T < 0 || (int64_t)T * s.top_k > kMaxRows)
            return set_error(ECF_EINVAL, "n_tokens must be in [0, %lld / top_k] (got %d)", (long long)kMaxRows, T);
        if (stats)
            std::memset(stats, 0, sizeof *stats);
        if (T == 0)
            return ECF_OK;
        if (!d_x || !d_out || !d_ws)
            return set_error(ECF_EINVAL, "x, out and workspace must be given");
        if ((a->d_router_w == nullptr) == (a->d_router_logits == nullptr))
            return set_error(ECF_EINVAL, "give exactly one of d_router_w and d_router_logits");
        if ((a->d_expert_ptrs == nullptr) == (a->cache == nullptr))
            return set_error(ECF_EINVAL, "give exactly one of d_expert_ptrs and cache");
        if ((uintptr_t)d_ws % 256)
            return set_error(ECF_EINVAL, "workspace must be 256-byte aligned");
        if ((uintptr_t)d_x % 16)
            return set_error(ECF_EINVAL, "x must be 16-byte aligned");
        const WsLayout wl = ws_layout(s, T);
        if (ws_bytes < wl.total)
            return set_error(ECF_ENOSPC, "workspace too small: %zu < %zu bytes for %d tokens", ws_bytes,
                             wl.total, T);
        const int path = pick_path(a, T);
        if (path == ECF_PATH_PREFILL && (s.w_dtype == ECF_F32 || s.inter % 128))
            return set_error(ECF_EUNSUPPORTED, "the prefill path needs bf16/MXFP4 weights and inter %% 128 == 0");
        hipStream_t stream = (hipStream_t)a->stream;
        char *ws = (char *)d_ws;
        BlobLayout lay;
        blob_layout(s, &lay);

        RouteOut ro;
        ro.idx = (int32_t *)(ws + wl.idx);
        ro.gate = (float *)(ws + wl.gate);
        ro.counts = (int32_t *)(ws + wl.counts);
        ro.offsets = (int32_t *)(ws + wl.offsets);
        ro.perm = (int32_t *)(ws + wl.perm);
        ro.pos = (int32_t *)(ws + wl.pos);
        ro.active = (int32_t *)(ws + wl.active);
        ro.n_active = (int32_t *)(ws + wl.n_active);
        ro.tiles = (int32_t *)(ws + wl.tiles);
        ro.n_tiles = (int32_t *)(ws + wl.n_tiles);
        ro.seg_counts = (int32_t *)(ws + wl.seg_counts);
        ro.seg_base = (int32_t *)(ws + wl.seg_base);

        const float *lg = a->d_router_logits;
        if (!lg) {
            float *dl = a->d_logits ? a->d_logits : (float *)(ws + wl.logits);
            if ((rc = launch_router_logits(s, d_x, a->d_router_w, T, dl, stream)) != ECF_OK)
                return rc;
            lg = dl;
        }
        // One token on the decode path, all experts resident, MXFP4 weights: the
        // down projection and the combine run as one kernel.
        const bool fused_down = !a->cache && path == ECF_PATH_DECODE && down_combine1_ok(s, T);
        // One token on the decode path, all experts resident, bf16 activations: the
        // gate/up GEMV derives the routing itself (no routing kernel).
        const bool route1 = !a->cache && path == ECF_PATH_DECODE && gateup_route1_ok(s, T);
        if (!route1 && (rc = launch_route(s, lg, T, ro, stream)) != ECF_OK)
            return rc;

        const float *host_part = nullptr;
        ExpertTables ex{a->d_expert_ptrs, lay};
        if (a->cache) {
            const uint64_t *tab = nullptr;
            if ((rc = cache_step(a, d_x, T, ro, wl, ws, lay, path, stats, &tab, &host_part)) != ECF_OK)
                return rc;
            ex.ptrs = tab;
        } else if (route1 || fused_down) {
            float *H = (float *)(ws + wl.hbuf);
            rc = route1 ? launch_decode_gateup_route1(s, ex, lg, d_x, ro, H, stream)
                        : launch_decode_gateup(s, ex, ro, d_x, T, H, stream);
            if (rc != ECF_OK)
                return rc;
            rc = fused_down
                     ? launch_decode_down_combine1(s, ex, ro, H, a->d_residual, d_out, a->d_out_act, stream)
                     : launch_decode_down(s, ex, ro, H, T, (float *)(ws + wl.ybuf), stream);
            if (rc != ECF_OK)
                return rc;
        } else if ((rc = launch_experts(s, ex, ro, d_x, T, wl, ws, path, stream)) != ECF_OK) {
            return rc;
        }
        if (!fused_down &&
            (rc = launch_combine(s, ex, ro, (const float *)(ws + wl.ybuf), T, a->d_residual, host_part, d_out,
                                 a->d_out_act, stream)) != ECF_OK)
            return rc;
        const int R = T * s.top_k;
        if (a->d_topk_idx)
            ECF_HIP_CHECK(hipMemcpyAsync(a->d_topk_idx, ro.idx, 4 * (size_t)R, hipMemcpyDeviceToDevice, stream));
        if (a->d_topk_gate)
            ECF_HIP_CHECK(hipMemcpyAsync(a->d_topk_gate, ro.gate, 4 * (size_t)R, hipMemcpyDeviceToDevice, stream));
        if (a->d_counts)
            ECF_HIP_CHECK(hipMemcpyAsync(a->d_counts, ro.counts, 4 * (size_t)s.n_experts,
                                         hipMemcpyDeviceToDevice, stream));
        if (a->d_perm)
            ECF_HIP_CHECK(hipMemcpyAsync(a->d_perm, ro.perm, 4 * (size_t)R, hipMemcpyDeviceToDevice, stream));
        if (stats)
            stats->path = path;
        return ECF_OK;
    } catch (const std::exception &e) {
        return set_error(ECF_EINVAL, "moe_layer_forward: %s", e.what());
    } catch (...) {
        return set_error(ECF_EINVAL, "moe_layer_forward: unknown failure");
    }
}

}  // namespace ecf

extern "C" int moe_layer_forward(const ecf_layer_args *a, const void *d_x, int32_t T, float *d_out,
                                 ecf_step_stats *stats)
{
    return forward_impl(a, d_x, T, d_out, stats, a ? a->d_ws : nullptr, a ? a->ws_bytes : 0);
}
