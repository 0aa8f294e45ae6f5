// Bandwidth profiler for the q* split: measures, on this machine, the pinned
// host -> device copy rate (B_P) and the rate at which the host expert threads
// consume expert weights, each alone and both at once.
//
// The split balances q copies against m - q host evaluations that share one
// host memory system, so the figures that matter are the ones measured while
// both run (techfeed.io summary of MarkTechPost, "FreeToken's three core
// mechanisms" / "Bandwidth-adaptive execution (q* policy)": the ratio comes
// from profiling the machine the engine runs on).  The host side is measured
// with the same expert FFN code the forward pass runs, so a CPU limited by its
// cores rather than its DRAM channels is measured as such.
#include <algorithm>
#include <atomic>
#include <cstdint>
#include <chrono>
#include <cstring>
#include <thread>
#include <vector>

#include "ecf_internal.h"
#include "host_ffn.h"

namespace ecf {
namespace {

using Clock = std::chrono::steady_clock;

double secs_since(Clock::time_point t0) { return std::chrono::duration<double>(Clock::now() - t0).count(); }

// Copies blob i % n into destination slot i % n_dst until `seconds` pass (or
// `stop` is set once at least one batch is done); bytes and seconds out.
int copy_loop(const void *const *h, int n, size_t S, char *d, int n_dst, hipStream_t st, double seconds,
              const std::atomic<bool> *stop, double *bytes, double *el)
{
    constexpr int kBatch = 4;
    const auto t0 = Clock::now();
    double b = 0.0;
    int i = 0;
    do {
        for (int j = 0; j < kBatch; ++j, ++i)
            ECF_HIP_CHECK(hipMemcpyAsync(d + (size_t)(i % n_dst) * S, h[i % n], S, hipMemcpyHostToDevice, st));
        ECF_HIP_CHECK(hipStreamSynchronize(st));
        b += (double)kBatch * S;
    } while (secs_since(t0) < seconds && !(stop && stop->load()));
    *bytes = b;
    *el = secs_since(t0);
    return ECF_OK;
}

// Host experts over blob i % n (one routed row each, as most host-assigned
// decode experts have) in rounds of n_round jobs until `seconds` pass.
int host_loop(HostPool &pool, const ecf_shape &s, const BlobLayout &lay, const void *const *h, int n,
              const void *x, float *y, double seconds, const std::atomic<bool> *stop, double *bytes, double *el)
{
    const int n_round = std::max(pool.size(), std::min(n, 2 * pool.size()));
    std::vector<HostExpertJob> jobs(n_round);
    const auto t0 = Clock::now();
    double b = 0.0;
    int at = 0;
    do {
        for (int j = 0; j < n_round; ++j, ++at) {
            jobs[j].expert = j;
            jobs[j].blob = h[at % n];
            jobs[j].rows.assign(1, j % s.top_k);  // token 0, slot j % k
        }
        const int rc = host_experts(pool, s, lay, jobs, x, 1, y);
        if (rc != ECF_OK)
            return rc;
        b += (double)n_round * (double)lay.bytes;
    } while (secs_since(t0) < seconds && !(stop && stop->load()));
    *bytes = b;
    *el = secs_since(t0);
    return ECF_OK;
}

// Plain streaming read of the blobs by the pool's threads (64-bit words).
double read_rate(HostPool &pool, const void *const *h, int n, size_t S, double seconds)
{
    const size_t words = S / 8, chunk = (size_t)1 << 18;  // 2 MB per task
    const size_t per_blob = (words + chunk - 1) / chunk;
    const int task_n = (int)(per_blob * n);
    std::vector<uint64_t> sink((size_t)task_n * 8, 0);  // one padded slot per task
    const auto t0 = Clock::now();
    double b = 0.0;
    do {
        pool.parallel_for(task_n, [&](int t) {
            const uint64_t *w = (const uint64_t *)h[t / per_blob];
            const size_t lo = (t % per_blob) * chunk, hi = std::min(words, lo + chunk);
            uint64_t acc0 = 0, acc1 = 0, acc2 = 0, acc3 = 0;
            size_t i = lo;
            for (; i + 4 <= hi; i += 4) {
                acc0 += w[i];
                acc1 += w[i + 1];
                acc2 += w[i + 2];
                acc3 += w[i + 3];
            }
            for (; i < hi; ++i)
                acc0 += w[i];
            sink[(size_t)t * 8] += acc0 + acc1 + acc2 + acc3;
        });
        b += (double)(words * 8) * n;
    } while (secs_since(t0) < seconds);
    volatile uint64_t keep = 0;
    for (uint64_t v : sink)
        keep = keep + v;
    (void)keep;
    return b / secs_since(t0) / 1e9;
}

}  // namespace
}  // namespace ecf

using namespace ecf;

extern "C" int ecf_bandwidth_profile(const ecf_shape *shape, int32_t n_blobs, const void *const *h_blobs,
                                     int32_t host_threads, void *d_buf, size_t d_buf_bytes, void *copy_stream,
                                     double seconds, ecf_bw_profile *out)
{
    try {
        if (!shape || !out || !h_blobs || n_blobs < 1 || !d_buf || host_threads < 0 || !(seconds > 0.0))
            return set_error(ECF_EINVAL, "ecf_bandwidth_profile: bad arguments");
        for (int32_t i = 0; i < n_blobs; ++i)
            if (!h_blobs[i])
                return set_error(ECF_EINVAL, "ecf_bandwidth_profile: blob %d is NULL", i);
        BlobLayout lay;
        const size_t S = ecf_expert_bytes(shape);
        if (S == 0)
            return ECF_EINVAL;  // ecf_expert_bytes set the message
        blob_layout(*shape, &lay);
        if (d_buf_bytes < S)
            return set_error(ECF_ENOSPC, "ecf_bandwidth_profile: device buffer %zu B < one expert (%zu B)",
                             d_buf_bytes, S);
        std::memset(out, 0, sizeof *out);
        const int n_dst = (int)std::min<size_t>(d_buf_bytes / S, 64);
        const int nt = host_threads > 0 ? host_threads
                                        : (int)std::min(16u, std::max(1u, std::thread::hardware_concurrency()));
        HostPool pool(nt);
        hipStream_t st = (hipStream_t)copy_stream;
        int dev = 0;
        ECF_HIP_CHECK(hipGetDevice(&dev));
        // one token of activations (small values) and its output rows
        std::vector<uint16_t> xb(shape->hidden, 0x3c00);  // bf16 / low half of f32: small
        std::vector<float> xf(shape->hidden, 0.01f);
        const void *x = shape->a_dtype == ECF_BF16 ? (const void *)xb.data() : (const void *)xf.data();
        std::vector<float> y((size_t)shape->top_k * shape->hidden);
        const double t1 = seconds / 4.0;

        double b, el;
        int rc;
        // warm both paths once, then each alone
        if ((rc = copy_loop(h_blobs, n_blobs, S, (char *)d_buf, n_dst, st, 0.0, nullptr, &b, &el)) ||
            (rc = host_loop(pool, *shape, lay, h_blobs, n_blobs, x, y.data(), 0.0, nullptr, &b, &el)))
            return rc;
        if ((rc = copy_loop(h_blobs, n_blobs, S, (char *)d_buf, n_dst, st, t1, nullptr, &b, &el)))
            return rc;
        out->b_p = b / el / 1e9;
        if ((rc = host_loop(pool, *shape, lay, h_blobs, n_blobs, x, y.data(), t1, nullptr, &b, &el)))
            return rc;
        out->b_cpu = b / el / 1e9;
        out->b_read = read_rate(pool, h_blobs, n_blobs, S, t1);

        // both at once: the copy loop on its own thread for as long as the host loop runs
        std::atomic<bool> stop{false};
        int crc = ECF_OK;
        double cb = 0.0, cel = 1.0;
        std::thread copier([&] {
            if (hipSetDevice(dev) != hipSuccess) {
                crc = set_error(ECF_EHIP, "ecf_bandwidth_profile: hipSetDevice failed");
                return;
            }
            crc = copy_loop(h_blobs, n_blobs, S, (char *)d_buf, n_dst, st, 1e9, &stop, &cb, &cel);
        });
        rc = host_loop(pool, *shape, lay, h_blobs, n_blobs, x, y.data(), t1, nullptr, &b, &el);
        stop.store(true);
        copier.join();
        if (rc != ECF_OK)
            return rc;
        if (crc != ECF_OK)  // the copier's message sits in its own thread's error slot
            return set_error(crc, "ecf_bandwidth_profile: the copy thread failed (HIP error)");
        out->b_p_conc = cb / cel / 1e9;
        out->b_cpu_conc = b / el / 1e9;
        out->b_h = out->b_p_conc + out->b_cpu_conc;
        out->host_threads = nt;
        return ECF_OK;
    } catch (...) {
        return set_error(ECF_EINVAL, "ecf_bandwidth_profile: failure");
    }
}
