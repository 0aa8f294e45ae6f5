// Internal declarations shared by the host-side sources of libecf.
#pragma once

#include <new>

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/ecf.h"

namespace ecf {

// ---- errors -------------------------------------------------------------------
int set_error(int code, const char *fmt, ...);
// Runs an entry point's body; no exception crosses the C ABI (host memory
// exhaustion -> ECF_ENOSPC, anything else -> ECF_EINVAL).
template <class F>
int guarded(const char *name, F &&f) noexcept
{
    try {
        return f();
    } catch (const std::bad_alloc &) {
        return set_error(ECF_ENOSPC, "%s: out of host memory", name);
    } catch (...) {
        return set_error(ECF_EINVAL, "%s: internal failure", name);
    }
}

#define ECF_HIP_CHECK(expr)                                                                   \
    do {                                                                                      \
        hipError_t _e = (expr);                                                               \
        if (_e != hipSuccess)                                                                 \
            return ::ecf::set_error(ECF_EHIP, "%s failed: %s (%s:%d)", #expr,                \
                                    hipGetErrorString(_e), __FILE__, __LINE__);               \
    } while (0)

// ---- profiling (event pairs around launches) ------------------------------------
struct ProfScope {
    ProfScope(const char *name, hipStream_t s);
    ~ProfScope();
    const char *name_;
    hipStream_t s_;
    hipEvent_t a_ = nullptr, b_ = nullptr;
};

// While set on a thread, ProfScope records nothing there (no events created):
// the allocation-free forward call sets it for its duration.
extern thread_local bool t_prof_quiet;

// The layer forward on an explicit workspace (moe_layer_forward passes the
// caller's, moe_layer_forward_noalloc the library's own device array).
int forward_impl(const ecf_layer_args *a, const void *d_x, int32_t T, float *d_out, ecf_step_stats *stats,
                 void *d_ws, size_t ws_bytes);

// ---- geometry ------------------------------------------------------------------
constexpr int64_t kMaxRows = (int64_t)1 << 26;  // n_tokens * top_k per call (row indices are 32-bit)
constexpr int kSortSeg = 1024;      // rows per segment of the multi-block counting sort
constexpr int kSmallRouteRows = 2048; // R up to this uses the single-block routing kernel
constexpr int kPrefillMT = 128;     // rows per prefill GEMM tile (bf16 weights)
#ifndef ECF_MX_BM
#define ECF_MX_BM 320                // rows per prefill GEMM tile (MXFP4 weights)
#endif
constexpr int kDecodeNT = 2;        // max rows per pass of the decode GEMV kernels

struct BlobLayout {
    size_t off[6];  // w_gate, w_up, w_down, s_gate, s_up, s_down
    size_t bytes;
};
bool blob_layout(const ecf_shape &s, BlobLayout *out);

// Workspace carve-up for up to T tokens.
struct WsLayout {
    size_t logits, idx, gate, counts, offsets, perm, pos, active, n_active, tiles, n_tiles,
        seg_counts, seg_base, ptrs, hbuf, ybuf, host_out, total;
};
WsLayout ws_layout(const ecf_shape &s, int32_t T);
int max_tiles(const ecf_shape &s, int32_t T);
// Rows per prefill GEMM tile for this shape; the routing kernels build the tile list with it.
inline int prefill_mt(const ecf_shape &s) { return s.w_dtype == ECF_MXFP4 ? ECF_MX_BM : kPrefillMT; }

// ---- kernel launchers (k_*.hip) -------------------------------------------------
struct RouteOut {
    int32_t *idx;
    float *gate;
    int32_t *counts, *offsets, *perm, *pos, *active, *n_active, *tiles, *n_tiles;
    int32_t *seg_counts, *seg_base;
};

int launch_router_logits(const ecf_shape &s, const void *x, const void *wr, int T, float *logits,
                         hipStream_t st);
int launch_route(const ecf_shape &s, const float *logits, int T, const RouteOut &o, hipStream_t st);

struct ExpertTables {
    const uint64_t *ptrs;  // [E] device blob addresses (0 = not evaluated on the GPU)
    BlobLayout lay;
};

int launch_decode_gateup(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const void *x,
                         int T, float *H, hipStream_t st);

int launch_decode_down(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const float *H,
                       int T, float *Y, hipStream_t st);
int launch_prefill_gemm1(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const void *x,
                         int T, uint16_t *H, hipStream_t st);
int launch_prefill_gemm2(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const uint16_t *H,
                         int T, float *Y, hipStream_t st);
// One token (T = 1, k <= 8, MXFP4 weights with bf16 activations): the down
// projection and the combine in one kernel, no Y in memory.
bool down_combine1_ok(const ecf_shape &s, int T);
// one token, bf16 activations, bf16 or MXFP4 weights: routing inside the gate/up GEMV
bool gateup_route1_ok(const ecf_shape &s, int T);
int launch_decode_gateup_route1(const ecf_shape &s, const ExpertTables &ex, const float *logits, const void *x,
                                const RouteOut &o, float *H, hipStream_t st);
int launch_decode_down_combine1(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const float *H,
                                const float *residual, float *out, void *out_act, hipStream_t st);
int launch_combine(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const float *Y, int T,
                   const float *residual, const float *host_part, float *out, void *out_act,
                   hipStream_t st);

}  // namespace ecf
