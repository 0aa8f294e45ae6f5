// Host-core expert FFNs: the CPU half of the bandwidth-adaptive split.
//
// techfeed summary of "Meet FreeToken" (MarkTechPost), section "Bandwidth-adaptive
// execution (q* policy)": the experts of a step's misses that are not copied are
// computed on the CPU directly from host memory, in parallel with the PCIe
// copies, using the host bandwidth the copies leave free.  leadeas blog, section
// "Using VRAM as a cache": a miss runs either on the CPU from host RAM or on the
// GPU after a transfer.
//
// Each host thread streams whole weight rows of one expert from the pinned pool
// (bf16 widened by a shift, exact) and applies each row to all of that expert's
// routed rows, so every weight byte is read once.  Phase 1 splits the
// gate/up rows of all host experts over the threads, phase 2 the down rows.
#include "host_ffn.h"

#include <immintrin.h>

#include <cmath>
#include <cstring>

namespace ecf {

// ---- thread pool ----------------------------------------------------------------

HostPool::HostPool(int n_threads)
{
    for (int i = 1; i < n_threads; ++i)
        th_.emplace_back([this] { worker(); });
}

HostPool::~HostPool()
{
    {
        std::lock_guard<std::mutex> g(mu_);
        stop_ = true;
        ++epoch_;
    }
    cv_.notify_all();
    for (auto &t : th_)
        t.join();
}

void HostPool::worker()
{
    uint64_t seen = 0;
    for (;;) {
        const std::function<void(int)> *fn;
        int total;
        {
            std::unique_lock<std::mutex> lk(mu_);
            cv_.wait(lk, [&] { return epoch_ != seen; });
            seen = epoch_;
            if (stop_)
                return;
            fn = fn_;
            total = total_;
        }
        for (int i = next_.fetch_add(1); i < total; i = next_.fetch_add(1))
            (*fn)(i);
        {
            std::lock_guard<std::mutex> g(mu_);
            if (--busy_ == 0)
                done_cv_.notify_all();
        }
    }
}

void HostPool::parallel_for(int n, const std::function<void(int)> &fn)
{
    if (n <= 0)
        return;
    {
        std::lock_guard<std::mutex> g(mu_);
        fn_ = &fn;
        total_ = n;
        next_.store(0);
        busy_ = (int)th_.size();
        ++epoch_;
    }
    cv_.notify_all();
    for (int i = next_.fetch_add(1); i < n; i = next_.fetch_add(1))
        fn(i);
    std::unique_lock<std::mutex> lk(mu_);
    done_cv_.wait(lk, [&] { return busy_ == 0; });
}

// ---- dot products ----------------------------------------------------------------

namespace {

constexpr int kRowsPerDot = 4;

inline float bf_to_f(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// out[r] = sum_c w[c] * xs[r][c], 16 partial sums per row (scalar build).
template <bool WBF>
void dots_scalar(const void *w, const float *const *xs, int nr, int n, float *out)
{
    for (int r = 0; r < nr; ++r) {
        float acc[16] = {};
        for (int c = 0; c < n; c += 16)
            for (int i = 0; i < 16; ++i) {
                const float wv = WBF ? bf_to_f(((const uint16_t *)w)[c + i]) : ((const float *)w)[c + i];
                acc[i] += wv * xs[r][c + i];
            }
        float s = 0.f;
        for (int i = 0; i < 16; ++i)
            s += acc[i];
        out[r] = s;
    }
}

__attribute__((target("avx2,fma"))) inline float hsum256(__m256 v)
{
    __m128 lo = _mm256_castps256_ps128(v), hi = _mm256_extractf128_ps(v, 1);
    lo = _mm_add_ps(lo, hi);
    lo = _mm_add_ps(lo, _mm_movehl_ps(lo, lo));
    lo = _mm_add_ss(lo, _mm_shuffle_ps(lo, lo, 1));
    return _mm_cvtss_f32(lo);
}

// Same sums with AVX2: two 8-wide accumulators per row = 16 partial sums.
template <bool WBF>
__attribute__((target("avx2,fma"))) void dots_avx2(const void *w, const float *const *xs, int nr, int n,
                                                   float *out)
{
    for (int r0 = 0; r0 < nr; r0 += kRowsPerDot) {
        const int m = nr - r0 < kRowsPerDot ? nr - r0 : kRowsPerDot;
        __m256 acc[kRowsPerDot][2];
        for (int r = 0; r < kRowsPerDot; ++r)
            acc[r][0] = acc[r][1] = _mm256_setzero_ps();
        for (int c = 0; c < n; c += 16) {
            __m256 w0, w1;
            if (WBF) {
                const uint16_t *p = (const uint16_t *)w + c;
                const __m128i a = _mm_loadu_si128((const __m128i *)p);
                const __m128i b = _mm_loadu_si128((const __m128i *)(p + 8));
                w0 = _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(a), 16));
                w1 = _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(b), 16));
            } else {
                w0 = _mm256_loadu_ps((const float *)w + c);
                w1 = _mm256_loadu_ps((const float *)w + c + 8);
            }
            for (int r = 0; r < m; ++r) {
                acc[r][0] = _mm256_fmadd_ps(w0, _mm256_loadu_ps(xs[r0 + r] + c), acc[r][0]);
                acc[r][1] = _mm256_fmadd_ps(w1, _mm256_loadu_ps(xs[r0 + r] + c + 8), acc[r][1]);
            }
        }
        for (int r = 0; r < m; ++r)
            out[r0 + r] = hsum256(_mm256_add_ps(acc[r][0], acc[r][1]));
    }
}

bool have_avx2()
{
    static const bool v = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma");
    return v;
}

template <bool WBF>
void dots(const void *w, const float *const *xs, int nr, int n, float *out)
{
    if (have_avx2())
        dots_avx2<WBF>(w, xs, nr, n, out);
    else
        dots_scalar<WBF>(w, xs, nr, n, out);
}

}  // namespace

int host_experts(HostPool &pool, const ecf_shape &s, const BlobLayout &lay,
                 const std::vector<HostExpertJob> &jobs, const void *x, int T, float *y)
{
    if (jobs.empty())
        return ECF_OK;
    if (s.w_dtype == ECF_MXFP4)
        return set_error(ECF_EUNSUPPORTED, "host experts: MXFP4 weights are not evaluated on the host");
    const int d = s.hidden, I = s.inter, k = s.top_k;
    const bool wbf = s.w_dtype == ECF_BF16;
    const size_t esz = wbf ? 2 : 4;
    // activations of every token in fp32
    std::vector<float> xf((size_t)T * d);
    if (s.a_dtype == ECF_BF16)
        for (size_t i = 0; i < xf.size(); ++i)
            xf[i] = bf_to_f(((const uint16_t *)x)[i]);
    else
        std::memcpy(xf.data(), x, xf.size() * 4);
    // h per job row
    std::vector<size_t> hoff(jobs.size() + 1, 0);
    for (size_t j = 0; j < jobs.size(); ++j)
        hoff[j + 1] = hoff[j] + jobs[j].rows.size() * (size_t)I;
    std::vector<float> h(hoff.back());

    constexpr int CH = 16;  // weight rows per task
    const int gu_chunks = (I + CH - 1) / CH, dn_chunks = (d + CH - 1) / CH;
    const int nj = (int)jobs.size();

    pool.parallel_for(nj * gu_chunks, [&](int task) {
        const HostExpertJob &jb = jobs[task / gu_chunks];
        const int nr = (int)jb.rows.size();
        std::vector<const float *> xs(nr);
        for (int r = 0; r < nr; ++r)
            xs[r] = xf.data() + (size_t)(jb.rows[r] / k) * d;
        std::vector<float> a(nr), b(nr);
        const char *wg = (const char *)jb.blob + lay.off[0], *wu = (const char *)jb.blob + lay.off[1];
        float *hj = h.data() + hoff[task / gu_chunks];
        const int i0 = (task % gu_chunks) * CH, i1 = std::min(I, i0 + CH);
        for (int i = i0; i < i1; ++i) {
            if (wbf) {
                dots<true>(wg + (size_t)i * d * esz, xs.data(), nr, d, a.data());
                dots<true>(wu + (size_t)i * d * esz, xs.data(), nr, d, b.data());
            } else {
                dots<false>(wg + (size_t)i * d * esz, xs.data(), nr, d, a.data());
                dots<false>(wu + (size_t)i * d * esz, xs.data(), nr, d, b.data());
            }
            for (int r = 0; r < nr; ++r)
                hj[(size_t)r * I + i] = a[r] / (1.0f + std::exp(-a[r])) * b[r];
        }
    });

    pool.parallel_for(nj * dn_chunks, [&](int task) {
        const HostExpertJob &jb = jobs[task / dn_chunks];
        const int nr = (int)jb.rows.size();
        const float *hj = h.data() + hoff[task / dn_chunks];
        std::vector<const float *> hs(nr);
        for (int r = 0; r < nr; ++r)
            hs[r] = hj + (size_t)r * I;
        std::vector<float> o(nr);
        const char *wd = (const char *)jb.blob + lay.off[2];
        const int o0 = (task % dn_chunks) * CH, o1 = std::min(d, o0 + CH);
        for (int oo = o0; oo < o1; ++oo) {
            if (wbf)
                dots<true>(wd + (size_t)oo * I * esz, hs.data(), nr, I, o.data());
            else
                dots<false>(wd + (size_t)oo * I * esz, hs.data(), nr, I, o.data());
            for (int r = 0; r < nr; ++r)
                y[(size_t)jb.rows[r] * d + oo] = o[r];
        }
    });
    return ECF_OK;
}

}  // namespace ecf
