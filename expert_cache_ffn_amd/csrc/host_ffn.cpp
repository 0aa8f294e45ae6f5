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
// and applies each row to all of that expert's routed rows, so every weight
// byte is read once.  Products are exact in every form (bf16 x bf16 pairs on
// AVX-512 BF16, otherwise bf16 / E2M1 x scale widened exactly to fp32), sums
// are fp32 with 16 or 32 independent partial sums per dot product.  Phase 1 splits the
// gate/up rows of all host experts over the threads, phase 2 the down rows.
#include "host_ffn.h"

#include <immintrin.h>

#include <chrono>
#include <cmath>
#include <cstdlib>
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
        stop_.store(true, std::memory_order_relaxed);
        epoch_.fetch_add(1, std::memory_order_release);
    }
    cv_.notify_all();
    for (auto &t : th_)
        t.join();
}

namespace {
// How long an idle worker spins before it sleeps: long enough to cover the
// gaps between the pool calls of one expert-cache layer-step (gate/up, down,
// host partial: a few microseconds apart), short enough that the workers are
// asleep while the calling thread waits on the GPU between layer-steps (with
// every core spinning, that thread's own wake-up was delayed: one token at a
// configured B_P/B_H of 0.4 went 24.3 -> 28.2 ms/step with a 0.5 ms spin).
constexpr auto kSpinFor = std::chrono::microseconds(50);
inline void cpu_relax() { _mm_pause(); }
}  // namespace

void HostPool::worker()
{
    uint64_t seen = 0;
    for (;;) {
        uint64_t e;
        int spins = 0;
        auto t0 = std::chrono::steady_clock::now();
        while ((e = epoch_.load(std::memory_order_acquire)) == seen) {
            if ((++spins & 63) != 0 || std::chrono::steady_clock::now() - t0 < kSpinFor) {
                cpu_relax();
                continue;
            }
            // The epoch is raised under mu_, so checking it under mu_ before
            // sleeping cannot miss a call.
            std::unique_lock<std::mutex> lk(mu_);
            cv_.wait(lk, [&] { return epoch_.load(std::memory_order_acquire) != seen; });
            spins = 0;
            t0 = std::chrono::steady_clock::now();
        }
        seen = e;
        if (stop_.load(std::memory_order_relaxed))
            return;
        run_tasks(*fn_.load(std::memory_order_relaxed), total_.load(std::memory_order_relaxed));
        busy_.fetch_sub(1, std::memory_order_release);
    }
}

void HostPool::run_tasks(const std::function<void(int)> &fn, int total)
{
    for (int i = next_.fetch_add(1); i < total; i = next_.fetch_add(1)) {
        try {
            fn(i);
        } catch (...) {
            std::lock_guard<std::mutex> g(mu_);
            if (!err_)
                err_ = std::current_exception();
        }
    }
}

void HostPool::parallel_for(int n, const std::function<void(int)> &fn)
{
    if (n <= 0)
        return;
    fn_.store(&fn, std::memory_order_relaxed);
    total_.store(n, std::memory_order_relaxed);
    next_.store(0, std::memory_order_relaxed);
    busy_.store((int)th_.size(), std::memory_order_relaxed);
    {
        std::lock_guard<std::mutex> g(mu_);
        epoch_.fetch_add(1, std::memory_order_release);
    }
    cv_.notify_all();
    run_tasks(fn, n);
    // every worker takes part in every call (it may find no index left), so
    // the call ends when all have checked out; fn must stay alive until then
    while (busy_.load(std::memory_order_acquire) != 0)
        cpu_relax();
    std::lock_guard<std::mutex> g(mu_);
    if (err_) {
        std::exception_ptr e = err_;
        err_ = nullptr;
        std::rethrow_exception(e);
    }
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

// Weight formats of a row: fp32, bf16, or MXFP4 (OCP MX v1.0: E2M1 elements,
// element 2i in the low nibble of byte i, one E8M0 scale per 32 elements).
enum { HF_F32 = 0, HF_BF16 = 1, HF_MX = 2 };

constexpr float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

// 2^(s - 127) built from its bits (s = 0: the subnormal 2^-127; 0xFF: NaN, as
// OCP MX v1.0 defines it).
inline float e8m0(uint8_t s)
{
    const uint32_t u = s == 0 ? 0x00400000u : s == 255 ? 0x7FC00000u : (uint32_t)s << 23;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// Weight c of a row (scalar build).
template <int WF>
inline float wval(const void *w, const uint8_t *sc, int c)
{
    if (WF == HF_BF16)
        return bf_to_f(((const uint16_t *)w)[c]);
    if (WF == HF_F32)
        return ((const float *)w)[c];
    const uint8_t b = ((const uint8_t *)w)[c >> 1];
    const int code = (c & 1) ? b >> 4 : b & 15;
    const float v = kE2M1[code & 7] * e8m0(sc[c >> 5]);
    return (code & 8) ? -v : v;
}

// out[r] = sum_c w[c] * xs[r][c], 16 partial sums per row (scalar build).
template <int WF>
void dots_scalar(const void *w, const uint8_t *sc, const float *const *xs, int nr, int n, float *out)
{
    for (int r = 0; r < nr; ++r) {
        float acc[16] = {};
        for (int c = 0; c < n; c += 16)
            for (int i = 0; i < 16; ++i)
                acc[i] += wval<WF>(w, sc, c + i) * xs[r][c + i];
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

// 8 E2M1 codes (int32 lanes) -> fp32 values times the block scale (exact).
__attribute__((target("avx2,fma"))) inline __m256 e2m1x8(__m256i code, __m256 scale)
{
    const __m256 mag = _mm256_permutevar8x32_ps(_mm256_loadu_ps(kE2M1), code);  // low 3 bits index
    const __m256 sgn = _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_srli_epi32(code, 3), 31));
    return _mm256_mul_ps(_mm256_xor_ps(mag, sgn), scale);
}

// Same sums with AVX2: two 8-wide accumulators per row = 16 partial sums.
// Byte offset of element c within a weight row.
template <int WF>
constexpr size_t wbytes(int c)
{
    return WF == HF_MX ? (size_t)c / 2 : (size_t)c * (WF == HF_BF16 ? 2 : 4);
}

template <int WF>
__attribute__((target("avx2,fma"))) void dots_avx2(const void *w, const uint8_t *sc, const float *const *xs,
                                                   int nr, int n, float *out)
{
    constexpr int STEP = WF == HF_MX ? 32 : 16;
    for (int r0 = 0; r0 < nr; r0 += kRowsPerDot) {
        const int m = nr - r0 < kRowsPerDot ? nr - r0 : kRowsPerDot;
        __m256 acc[kRowsPerDot][2];
        for (int r = 0; r < kRowsPerDot; ++r)
            acc[r][0] = acc[r][1] = _mm256_setzero_ps();
        for (int c = 0; c < n; c += STEP) {
            _mm_prefetch((const char *)w + wbytes<WF>(c) + 1024, _MM_HINT_T0);  // 1 KB ahead
            __m256 wv[4];
            if (WF == HF_MX) {
                const __m128i bytes = _mm_loadu_si128((const __m128i *)((const uint8_t *)w + c / 2));
                const __m128i lo = _mm_and_si128(bytes, _mm_set1_epi8(0x0f));
                const __m128i hi = _mm_and_si128(_mm_srli_epi16(bytes, 4), _mm_set1_epi8(0x0f));
                const __m128i e0 = _mm_unpacklo_epi8(lo, hi), e1 = _mm_unpackhi_epi8(lo, hi);
                const __m256 scale = _mm256_set1_ps(e8m0(sc[c / 32]));
                wv[0] = e2m1x8(_mm256_cvtepu8_epi32(e0), scale);
                wv[1] = e2m1x8(_mm256_cvtepu8_epi32(_mm_srli_si128(e0, 8)), scale);
                wv[2] = e2m1x8(_mm256_cvtepu8_epi32(e1), scale);
                wv[3] = e2m1x8(_mm256_cvtepu8_epi32(_mm_srli_si128(e1, 8)), scale);
            } else if (WF == HF_BF16) {
                const uint16_t *p = (const uint16_t *)w + c;
                const __m128i a = _mm_loadu_si128((const __m128i *)p);
                const __m128i b = _mm_loadu_si128((const __m128i *)(p + 8));
                wv[0] = _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(a), 16));
                wv[1] = _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(b), 16));
            } else {
                wv[0] = _mm256_loadu_ps((const float *)w + c);
                wv[1] = _mm256_loadu_ps((const float *)w + c + 8);
            }
            for (int r = 0; r < m; ++r) {
                const float *xp = xs[r0 + r] + c;
                for (int v = 0; v < STEP / 8; ++v)
                    acc[r][v & 1] = _mm256_fmadd_ps(wv[v], _mm256_loadu_ps(xp + 8 * v), acc[r][v & 1]);
            }
        }
        for (int r = 0; r < m; ++r)
            out[r0 + r] = hsum256(_mm256_add_ps(acc[r][0], acc[r][1]));
    }
}

// AVX-512: 16-wide, two accumulators per row (32 partial sums).  bf16 weights
// against bf16 activations use VDPBF16PS (pairs of exact bf16 products summed
// in fp32); everything else widens the weights to fp32 and uses FMAs.  xb
// (nullable) holds the same rows as xs in bf16.
constexpr float kE2M1Signed[16] = {0.0f,  0.5f,  1.0f,  1.5f,  2.0f,  3.0f,  4.0f,  6.0f,
                                   -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f};

template <int WF>
__attribute__((target("avx512f,avx512bw,avx512vl,avx512bf16"))) void dots_avx512(
    const void *w, const uint8_t *sc, const float *const *xs, const uint16_t *const *xb, int nr, int n,
    float *out)
{
    const bool dp = WF == HF_BF16 && xb != nullptr;
    const __m512 tab = _mm512_loadu_ps(kE2M1Signed);
    for (int r0 = 0; r0 < nr; r0 += kRowsPerDot) {
        const int m = nr - r0 < kRowsPerDot ? nr - r0 : kRowsPerDot;
        __m512 acc[kRowsPerDot][2];
        for (int r = 0; r < kRowsPerDot; ++r)
            acc[r][0] = acc[r][1] = _mm512_setzero_ps();
        for (int c = 0; c < n; c += 32) {  // n is a multiple of 32
            // the weight stream 1 KB ahead (past a row's end it touches the next row;
            // a prefetch never faults)
            _mm_prefetch((const char *)w + wbytes<WF>(c) + 1024, _MM_HINT_T0);
            if (dp) {
                const __m512i wv = _mm512_loadu_si512((const void *)((const uint16_t *)w + c));
                for (int r = 0; r < m; ++r) {
                    const __m512i xv = _mm512_loadu_si512((const void *)(xb[r0 + r] + c));
                    acc[r][(c >> 5) & 1] = _mm512_dpbf16_ps(acc[r][(c >> 5) & 1], (__m512bh)wv, (__m512bh)xv);
                }
                continue;
            }
            __m512 wv[2];
            if (WF == HF_MX) {
                const __m128i bytes = _mm_loadu_si128((const __m128i *)((const uint8_t *)w + c / 2));
                const __m128i lo = _mm_and_si128(bytes, _mm_set1_epi8(0x0f));
                const __m128i hi = _mm_and_si128(_mm_srli_epi16(bytes, 4), _mm_set1_epi8(0x0f));
                const __m512 scale = _mm512_set1_ps(e8m0(sc[c / 32]));
                wv[0] = _mm512_mul_ps(_mm512_permutexvar_ps(_mm512_cvtepu8_epi32(_mm_unpacklo_epi8(lo, hi)), tab), scale);
                wv[1] = _mm512_mul_ps(_mm512_permutexvar_ps(_mm512_cvtepu8_epi32(_mm_unpackhi_epi8(lo, hi)), tab), scale);
            } else if (WF == HF_BF16) {
                const __m256i a = _mm256_loadu_si256((const __m256i *)((const uint16_t *)w + c));
                const __m256i b = _mm256_loadu_si256((const __m256i *)((const uint16_t *)w + c + 16));
                wv[0] = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(a), 16));
                wv[1] = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(b), 16));
            } else {
                wv[0] = _mm512_loadu_ps((const float *)w + c);
                wv[1] = _mm512_loadu_ps((const float *)w + c + 16);
            }
            for (int r = 0; r < m; ++r) {
                const float *xp = xs[r0 + r] + c;
                acc[r][0] = _mm512_fmadd_ps(wv[0], _mm512_loadu_ps(xp), acc[r][0]);
                acc[r][1] = _mm512_fmadd_ps(wv[1], _mm512_loadu_ps(xp + 16), acc[r][1]);
            }
        }
        for (int r = 0; r < m; ++r)
            out[r0 + r] = _mm512_reduce_add_ps(_mm512_add_ps(acc[r][0], acc[r][1]));
    }
}

enum Isa { ISA_SCALAR = 0, ISA_AVX2 = 1, ISA_AVX512 = 2 };

// The widest instruction set this CPU has (AVX-512 with BF16 dot products, else
// AVX2 + FMA, else scalar); ECF_HOST_ISA=avx2 or =scalar asks for a narrower one.
Isa host_isa()
{
    static const Isa hw = [] {
        if (__builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
            __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("avx512bf16"))
            return ISA_AVX512;
        if (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma"))
            return ISA_AVX2;
        return ISA_SCALAR;
    }();
    const char *e = std::getenv("ECF_HOST_ISA");
    if (e && !std::strcmp(e, "scalar"))
        return ISA_SCALAR;
    if (e && !std::strcmp(e, "avx2") && hw >= ISA_AVX2)
        return ISA_AVX2;
    return hw;
}

template <int WF>
void dots(Isa isa, const void *w, const uint8_t *sc, const float *const *xs, const uint16_t *const *xb, int nr,
          int n, float *out)
{
    if (isa == ISA_AVX512)
        dots_avx512<WF>(w, sc, xs, xb, nr, n, out);
    else if (isa == ISA_AVX2)
        dots_avx2<WF>(w, sc, xs, nr, n, out);
    else
        dots_scalar<WF>(w, sc, xs, nr, n, out);
}

// Row i of a weight section (element count n per row) and its scale row.
struct RowRef {
    const char *w;
    const uint8_t *sc;
};

inline RowRef row_of(const void *blob, size_t off_w, size_t off_s, int wf, int i, int n)
{
    const char *b = (const char *)blob;
    if (wf == HF_MX)
        return {b + off_w + (size_t)i * n / 2, (const uint8_t *)b + off_s + (size_t)i * (n / 32)};
    return {b + off_w + (size_t)i * n * (wf == HF_BF16 ? 2 : 4), nullptr};
}

void dots_any(Isa isa, int wf, RowRef row, const float *const *xs, const uint16_t *const *xb, int nr, int n,
              float *out)
{
    if (wf == HF_MX)
        dots<HF_MX>(isa, row.w, row.sc, xs, xb, nr, n, out);
    else if (wf == HF_BF16)
        dots<HF_BF16>(isa, row.w, row.sc, xs, xb, nr, n, out);
    else
        dots<HF_F32>(isa, row.w, row.sc, xs, xb, nr, n, out);
}

}  // namespace

// Per-thread scratch of the expert tasks, reused across tasks and calls.  Each
// thread that runs a task enters this function, so its copy is constructed
// there on first use and destroyed when the thread ends.
struct Scratch {
    std::vector<const float *> xs;
    std::vector<const uint16_t *> xb;
    std::vector<float> a, b;
};
static Scratch &scratch()
{
    static thread_local Scratch s;
    return s;
}

int host_experts(HostPool &pool, const ecf_shape &s, const BlobLayout &lay,
                 const std::vector<HostExpertJob> &jobs, const void *x, int T, float *y)
{
    if (jobs.empty())
        return ECF_OK;
    const int d = s.hidden, I = s.inter, k = s.top_k;
    const int wf = s.w_dtype == ECF_MXFP4 ? HF_MX : s.w_dtype == ECF_BF16 ? HF_BF16 : HF_F32;
    const Isa isa = host_isa();
    const bool xbf = s.a_dtype == ECF_BF16;
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

    // weight rows per task: 16 gate + 16 up rows (256 KB of bf16 at d 4096), 64
    // down rows (128 KB at I 1024), so a task's fixed costs stay small
    constexpr int CH = 16, CHD = 64;
    const int gu_chunks = (I + CH - 1) / CH, dn_chunks = (d + CHD - 1) / CHD;
    const int nj = (int)jobs.size();
    pool.parallel_for(nj * gu_chunks, [&](int task) {
        const HostExpertJob &jb = jobs[task / gu_chunks];
        const int nr = (int)jb.rows.size();
        Scratch &sc = scratch();
        sc.xs.resize(nr);
        sc.xb.resize(nr);
        sc.a.resize(nr);
        sc.b.resize(nr);
        std::vector<const float *> &xs = sc.xs;
        std::vector<const uint16_t *> &xb = sc.xb;
        for (int r = 0; r < nr; ++r) {
            const size_t t = (size_t)(jb.rows[r] / k);
            xs[r] = xf.data() + t * d;
            xb[r] = xbf ? (const uint16_t *)x + t * d : nullptr;
        }
        const uint16_t *const *xbp = xbf ? xb.data() : nullptr;
        std::vector<float> &a = sc.a, &b = sc.b;
        float *hj = h.data() + hoff[task / gu_chunks];
        const int i0 = (task % gu_chunks) * CH, i1 = std::min(I, i0 + CH);
        for (int i = i0; i < i1; ++i) {
            dots_any(isa, wf, row_of(jb.blob, lay.off[0], lay.off[3], wf, i, d), xs.data(), xbp, nr, d, a.data());
            dots_any(isa, wf, row_of(jb.blob, lay.off[1], lay.off[4], wf, i, d), xs.data(), xbp, nr, d, b.data());
            for (int r = 0; r < nr; ++r)
                hj[(size_t)r * I + i] = a[r] / (1.0f + std::exp(-a[r])) * b[r];
        }
    });

    pool.parallel_for(nj * dn_chunks, [&](int task) {
        const HostExpertJob &jb = jobs[task / dn_chunks];
        const int nr = (int)jb.rows.size();
        const float *hj = h.data() + hoff[task / dn_chunks];
        Scratch &sc = scratch();
        sc.xs.resize(nr);
        sc.a.resize(nr);
        std::vector<const float *> &hs = sc.xs;
        for (int r = 0; r < nr; ++r)
            hs[r] = hj + (size_t)r * I;
        std::vector<float> &o = sc.a;
        const int o0 = (task % dn_chunks) * CHD, o1 = std::min(d, o0 + CHD);
        for (int oo = o0; oo < o1; ++oo) {
            dots_any(isa, wf, row_of(jb.blob, lay.off[2], lay.off[5], wf, oo, I), hs.data(), nullptr, nr, I,
                     o.data());
            for (int r = 0; r < nr; ++r)
                y[(size_t)jb.rows[r] * d + oo] = o[r];
        }
    });
    return ECF_OK;
}

}  // namespace ecf
