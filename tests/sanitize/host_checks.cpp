// Host-side checks of libecf's CPU code under the compiler's sanitizers
// (AddressSanitizer + UndefinedBehaviorSanitizer in one build, ThreadSanitizer
// in another): the shared LRU cache and its elastic resize, the q* split and
// the host expert FFN on its thread pool, all through the C ABI, and the thread
// pool itself through its internal header.  No GPU is touched: the GPU kernel
// launchers are replaced by stubs (stubs.cpp) that are never called, and no
// call below reaches a HIP runtime function.
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <set>
#include <stdexcept>
#include <thread>
#include <vector>

#include "ecf.h"
#include "../../expert_cache_ffn_amd/csrc/host_ffn.h"

static int g_fail = 0;
#define CHECK(c)                                                                  \
    do {                                                                          \
        if (!(c)) {                                                               \
            std::fprintf(stderr, "CHECK failed at %s:%d: %s\n", __FILE__, __LINE__, #c); \
            ++g_fail;                                                             \
        }                                                                         \
    } while (0)

// q*: always floor or ceil of m * b_p / b_h, in [0, m]
static void check_qstar()
{
    const double ratios[] = {0.0, 0.05, 0.186, 0.25, 0.4, 0.68, 0.999, 1.0, 1.5};
    for (double r : ratios)
        for (int m = 0; m <= 300; ++m) {
            const int q = qstar_split(m, r * 100.0, 100.0);
            const double x = m * std::min(r, 1.0);
            CHECK(q >= 0 && q <= m);
            CHECK(q == (int)std::floor(x) || q == (int)std::ceil(x));
        }
    CHECK(qstar_split(-1, 1, 2) < 0);
    CHECK(qstar_split(3, 1, 0) < 0);
    CHECK(qstar_split(3, NAN, 2) < 0);
}

// random lookups, binds and resizes over many layers; the cache's own view
// (slot_of, availability, counters) must stay consistent
static void check_cache(unsigned seed)
{
    const int L = 7, E = 23, max_slots = 40;
    std::vector<char> dev(1);  // slot memory is never touched on the host
    ecf_cache *c = nullptr;
    CHECK(ecf_cache_create(L, E, 30, max_slots, 1, dev.data(), nullptr, 2, &c) == ECF_OK);
    std::mt19937 rng(seed);
    int64_t lookups = 0, hits = 0, inserts = 0;
    for (int it = 0; it < 4000; ++it) {
        if (rng() % 97 == 0) {
            const int n = (int)(rng() % (max_slots + 1));
            CHECK(ecf_cache_resize(c, n) == ECF_OK);
            continue;
        }
        const int layer = (int)(rng() % L);
        std::set<int32_t> pick;
        const int n = 1 + (int)(rng() % 9);
        while ((int)pick.size() < n)
            pick.insert((int32_t)(rng() % E));
        std::vector<int32_t> ex(pick.begin(), pick.end()), slots(ex.size());
        CHECK(expert_cache_lookup(c, layer, ex.data(), (int32_t)ex.size(), slots.data()) == ECF_OK);
        lookups += (int64_t)ex.size();
        std::vector<int32_t> miss;
        for (size_t i = 0; i < ex.size(); ++i) {
            if (slots[i] >= 0) {
                ++hits;
                CHECK(ecf_cache_slot_of(c, layer, ex[i]) == slots[i]);
            } else {
                miss.push_back(ex[i]);
            }
        }
        const int avail = ecf_cache_available(c);
        CHECK(avail >= 0);
        const int q = std::min<int>((int)miss.size(), (int)(rng() % 6));
        std::vector<int32_t> got(q), victims(q);
        const int rc = expert_cache_evict(c, layer, miss.data(), q, got.data(), victims.data());
        if (q <= avail) {
            CHECK(rc == ECF_OK);
            inserts += q;
            for (int i = 0; i < q; ++i) {
                CHECK(ecf_cache_slot_of(c, layer, miss[i]) == got[i]);
                if (victims[i] >= 0)
                    CHECK(ecf_cache_slot_of(c, victims[i] / E, victims[i] % E) == -1);
            }
        } else {
            CHECK(rc == ECF_ENOSPC);
        }
        // no two pairs share a slot
        std::set<int32_t> used;
        for (int l = 0; l < L; ++l)
            for (int e = 0; e < E; ++e) {
                const int32_t s = ecf_cache_slot_of(c, l, e);
                if (s >= 0)
                    CHECK(used.insert(s).second);
            }
    }
    ecf_cache_stats st;
    CHECK(ecf_cache_get_stats(c, &st) == ECF_OK);
    CHECK(st.lookups == lookups && st.hits == hits && st.misses == lookups - hits && st.inserts == inserts);
    // an evict with no open layer-step, a repeated expert, a bad layer
    int32_t e3[2] = {3, 3}, sl[2];
    CHECK(ecf_cache_resize(c, 10) == ECF_OK);
    CHECK(expert_cache_evict(c, 0, e3, 1, sl, nullptr) == ECF_ESTATE);
    CHECK(expert_cache_lookup(c, 0, e3, 0, sl) == ECF_OK);
    CHECK(expert_cache_evict(c, 0, e3, 2, sl, nullptr) == ECF_EINVAL);
    CHECK(expert_cache_lookup(c, L, e3, 1, sl) == ECF_EINVAL);
    ecf_cache_destroy(c);
}

static uint16_t to_bf16(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// the host expert FFN over its thread pool: the same rows with 1 and with 8
// threads give identical outputs (each row's sums run in a fixed order), for
// fp32, bf16 and MXFP4 weights; bad rows are refused
static void check_host_experts(int w_dtype)
{
    const int d = 512, I = 256, E = 5, k = 2, T = 37;
    ecf_shape s{d, I, E, k, w_dtype, w_dtype == ECF_F32 ? ECF_F32 : ECF_BF16, 1};
    const size_t B = ecf_expert_bytes(&s);
    CHECK(B > 0);
    std::mt19937 rng(11 + w_dtype);
    std::vector<std::vector<uint8_t>> blobs(E, std::vector<uint8_t>(B));
    size_t off[6];
    CHECK(ecf_expert_layout(&s, off) == ECF_OK);
    std::normal_distribution<float> nd(0.f, 0.02f);
    for (auto &b : blobs) {
        if (w_dtype == ECF_F32) {
            float *w = (float *)b.data();
            for (size_t i = 0; i < B / 4; ++i)
                w[i] = nd(rng);
        } else if (w_dtype == ECF_BF16) {
            uint16_t *w = (uint16_t *)b.data();
            for (size_t i = 0; i < B / 2; ++i)
                w[i] = to_bf16(nd(rng));
        } else {
            for (size_t i = 0; i < off[3]; ++i)
                b[i] = (uint8_t)rng();
            for (size_t i = off[3]; i < B; ++i)
                b[i] = (uint8_t)(118 + rng() % 6);  // scales 2^-9 .. 2^-4
        }
    }
    std::vector<uint8_t> x((size_t)T * d * (w_dtype == ECF_F32 ? 4 : 2));
    std::normal_distribution<float> nx(0.f, 1.f);
    for (int i = 0; i < T * d; ++i) {
        if (w_dtype == ECF_F32)
            ((float *)x.data())[i] = nx(rng);
        else
            ((uint16_t *)x.data())[i] = to_bf16(nx(rng));
    }
    std::vector<const void *> bp;
    for (auto &b : blobs)
        bp.push_back(b.data());
    std::vector<int32_t> n_rows(E, 0), rows;
    std::vector<std::vector<int32_t>> per(E);
    for (int f = 0; f < T * k; ++f)
        per[f % E].push_back(f);
    for (int e = 0; e < E; ++e) {
        n_rows[e] = (int32_t)per[e].size();
        rows.insert(rows.end(), per[e].begin(), per[e].end());
    }
    std::vector<float> y1((size_t)T * k * d, 0.f), y8((size_t)T * k * d, 0.f);
    CHECK(ecf_host_experts(&s, E, bp.data(), n_rows.data(), rows.data(), x.data(), T, y1.data(), 1) == ECF_OK);
    CHECK(ecf_host_experts(&s, E, bp.data(), n_rows.data(), rows.data(), x.data(), T, y8.data(), 8) == ECF_OK);
    CHECK(std::memcmp(y1.data(), y8.data(), y1.size() * 4) == 0);
    bool finite = true;
    for (float v : y1)
        finite &= std::isfinite(v);
    CHECK(finite);
    std::vector<int32_t> bad = rows;
    bad[3] = T * k;  // one row past the end
    CHECK(ecf_host_experts(&s, E, bp.data(), n_rows.data(), bad.data(), x.data(), T, y8.data(), 4) == ECF_EINVAL);
}

// The host thread pool on its own: thousands of back-to-back calls of every
// size from 0 to 64 (the workers spin between them), pauses long enough for
// them to fall asleep, and calls in which a task throws (rethrown once per
// call, the pool usable afterwards).
static void check_pool()
{
    for (int nt : {1, 3, 8}) {
        ecf::HostPool pool(nt);
        std::vector<std::atomic<int>> hit(64);
        for (int it = 0; it < 3000; ++it) {
            const int n = it % 65;
            for (auto &h : hit)
                h.store(0, std::memory_order_relaxed);
            pool.parallel_for(n, [&](int i) { hit[i].fetch_add(1, std::memory_order_relaxed); });
            bool ok = true;
            for (int i = 0; i < 64; ++i)
                ok = ok && hit[i].load(std::memory_order_relaxed) == (i < n ? 1 : 0);
            CHECK(ok);
            if (it % 1000 == 999)
                std::this_thread::sleep_for(std::chrono::milliseconds(5));
        }
        int caught = 0;
        for (int it = 0; it < 20; ++it) {
            try {
                pool.parallel_for(40, [&](int i) {
                    if (i == 7 + it % 3)
                        throw std::runtime_error("task");
                });
            } catch (const std::runtime_error &) {
                ++caught;
            }
        }
        CHECK(caught == 20);
        std::atomic<int> sum{0};
        pool.parallel_for(100, [&](int i) { sum.fetch_add(i, std::memory_order_relaxed); });
        CHECK(sum.load() == 4950);
    }
}

int main()
{
    check_pool();
    check_qstar();
    for (unsigned seed = 1; seed <= 3; ++seed)
        check_cache(seed);
    check_host_experts(ECF_F32);
    check_host_experts(ECF_BF16);
    check_host_experts(ECF_MXFP4);
    if (g_fail) {
        std::fprintf(stderr, "%d check(s) failed\n", g_fail);
        return 1;
    }
    std::printf("host checks passed\n");
    return 0;
}
