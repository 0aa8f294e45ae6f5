// Host-core evaluation of experts assigned to the CPU by the q* split.
#pragma once

#include <atomic>
#include <condition_variable>
#include <cstdint>
#include <exception>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "ecf_internal.h"

namespace ecf {

// Fixed pool of worker threads; parallel_for runs fn(0..n-1) on the workers
// and the calling thread and returns when every index is done.  Idle workers
// spin on the call counter for about 50 us before they sleep on the condition
// variable, so back-to-back calls (an expert-cache layer-step makes three, a
// few microseconds apart) start without a thread wake-up; the caller spins for
// the last tasks to end.
class HostPool {
public:
    explicit HostPool(int n_threads);
    ~HostPool();
    int size() const { return (int)th_.size() + 1; }
    // fn(0..n-1) over the pool and the calling thread; returns once every call
    // has ended.  The first exception a call throws is rethrown here, after
    // the other calls have finished.
    void parallel_for(int n, const std::function<void(int)> &fn);

private:
    void worker();
    void run_tasks(const std::function<void(int)> &fn, int total);
    std::exception_ptr err_;  // under mu_
    std::vector<std::thread> th_;
    std::mutex mu_;
    std::condition_variable cv_;
    // Published before epoch_ is raised (release) and read after it is seen
    // (acquire): the call's function and size.
    std::atomic<const std::function<void(int)> *> fn_{nullptr};
    std::atomic<int> total_{0};
    std::atomic<int> next_{0};     // next index to run
    std::atomic<int> busy_{0};     // workers still in the current call
    std::atomic<uint64_t> epoch_{0};  // raised (under mu_) once per call and at shutdown
    std::atomic<bool> stop_{false};
};

struct HostExpertJob {
    int expert;
    const void *blob;       // pinned host blob of this (layer, expert)
    std::vector<int> rows;  // flat routed rows f = t*k + j sent to this expert
};

// y[f][:] = W_down . (silu(W_gate . x[t]) * (W_up . x[t])) for every row f of
// every job, t = f / k.  x: host [T][d] in a_dtype; weights fp32 or bf16.
// Math in fp32 with 16 independent partial sums per dot product.
int host_experts(HostPool &pool, const ecf_shape &s, const BlobLayout &lay,
                 const std::vector<HostExpertJob> &jobs, const void *x, int T, float *y);

}  // namespace ecf
