// Allocation-free variant of the layer forward: the workspace (routing
// tables, h and y rows, host partial) lives in a file-scope device array of
// the library instead of caller memory, for callers that cannot allocate.
#include <mutex>

#include "ecf_internal.h"

namespace ecf {
namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;  // 32 MiB per GPU, held until the process ends
constexpr int kMaxDevices = 64;

// The workspace of moe_layer_forward_noalloc.  In host code this name is only
// a host-side stand-in: kernels receive the device address that
// hipGetSymbolAddress returns for it (one copy per GPU).
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up once
// per device with that device current.
int scratch_ptr(void **out)
{
    int dev = -1;
    ECF_HIP_CHECK(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices)
        return set_error(ECF_EUNSUPPORTED, "moe_layer_forward_noalloc: device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        ECF_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p || (uintptr_t)p % 256)
            return set_error(ECF_EHIP, "moe_layer_forward_noalloc: bad scratch address %p", p);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ECF_OK;
}

struct QuietProfile {
    QuietProfile() { t_prof_quiet = true; }
    ~QuietProfile() { t_prof_quiet = false; }
};

}  // namespace
}  // namespace ecf

using namespace ecf;

extern "C" size_t ecf_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int moe_layer_forward_noalloc(const ecf_layer_args *a, const void *d_x, int32_t n_tokens,
                                         float *d_out, ecf_step_stats *stats)
{
    return guarded("moe_layer_forward_noalloc", [&]() -> int {
        if (!a)
            return set_error(ECF_EINVAL, "moe_layer_forward_noalloc: NULL args");
        if (a->cache)
            return set_error(ECF_EUNSUPPORTED,
                             "moe_layer_forward_noalloc: all-resident experts only (cache mode stages "
                             "routing through pinned host buffers it allocates)");
        if (n_tokens > 0 && n_tokens * (int64_t)a->shape.top_k <= (int64_t)1 << 26) {
            const size_t need = ecf_workspace_bytes(&a->shape, n_tokens);
            if (need > kScratchBytes)
                return set_error(ECF_ENOSPC,
                                 "moe_layer_forward_noalloc: %d tokens need %zu workspace bytes, above the "
                                 "%zu-byte scratch",
                                 n_tokens, need, kScratchBytes);
        }
        void *ws = nullptr;
        int rc = scratch_ptr(&ws);
        if (rc != ECF_OK)
            return rc;
        QuietProfile quiet;
        return forward_impl(a, d_x, n_tokens, d_out, stats, ws, kScratchBytes);
    });
}
